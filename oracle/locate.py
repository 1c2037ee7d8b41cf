"""One-byte-at-a-time view of the exchange, for sampled checks at full size.

TEST INFRASTRUCTURE ONLY.  Given the count matrix, answers "which input byte
lands at target byte (d, offset)?" without running the whole exchange, by
walking the sources of destination d in ascending order (the receive side is
packed by source) and, inside source s's slab, skipping the segments it
addresses to lower-numbered destinations (the send side is packed by
destination).  Same reading as :mod:`oracle.brute`, written per byte.
"""
from __future__ import annotations


def source_of(counts, d: int, offset: int, elem_size: int, in_slab: int):
    """Absolute input byte index feeding target byte ``d*tgt_slab + offset``.

    Returns None when ``offset`` lies past everything destination d receives
    (that byte keeps its old value).
    """
    P = len(counts)
    start = 0
    for s in range(P):
        n = int(counts[s][d]) * elem_size
        if offset < start + n:
            skip = sum(int(counts[s][dd]) * elem_size for dd in range(d))
            return s * in_slab + skip + (offset - start)
        start += n
    return None
