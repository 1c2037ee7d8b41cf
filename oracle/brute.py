"""Pure-Python brute force of the exchange, for tiny P (TEST INFRASTRUCTURE ONLY).

Independent of the C oracle and of the HIP library.  Each destination slab is
rebuilt by concatenating, over sources s in ascending order, the byte string
that source s addressed to it; source s's string for destination d is found by
skipping the strings s addressed to every lower-numbered destination.  This is
the reading of the five-operand all_to_all_v of the PyPTO
"LowerL2TensorCollectives Pass" page (input packed by destination, target
packed by source), with counts in elements as on the "vccl alltoallv dev log"
page (section 5: counts scaled by the type size).
"""
from __future__ import annotations


def exchange(input_slabs: list[bytes], target_slabs: list[bytes],
             counts: list[list[int]], elem_size: int) -> list[bytes]:
    """Return the new target slabs (same lengths as ``target_slabs``)."""
    P = len(input_slabs)
    pieces: dict[tuple[int, int], bytes] = {}
    for s in range(P):
        pos = 0
        for d in range(P):
            n = counts[s][d] * elem_size
            pieces[(s, d)] = input_slabs[s][pos:pos + n]
            pos += n
    out = []
    for d in range(P):
        received = b"".join(pieces[(s, d)] for s in range(P))
        old = target_slabs[d]
        out.append(received + old[len(received):])
    return out


def exchange_blocked(input_slabs: list[bytes], target_slabs: list[bytes],
                     counts: list[list[int]], elem_size: int, nblk: int) -> list[bytes]:
    """The blocked exchange by byte concatenation.

    Source slab s is read as nblk equal block-rows; each block-row lists the
    sub-blocks for destinations 0..P-1 in order, sub-block d being
    counts[s][d] / nblk elements.  Destination d receives, for s ascending,
    the nblk sub-blocks of s's segment in block-row order.
    """
    P = len(input_slabs)
    pieces: dict[tuple[int, int], bytes] = {}
    for s in range(P):
        subs = [counts[s][d] * elem_size // nblk for d in range(P)]
        row = sum(subs)                      # bytes per block-row
        parts = {d: b"" for d in range(P)}
        for a in range(nblk):
            block = input_slabs[s][a * row:(a + 1) * row]
            pos = 0
            for d in range(P):
                parts[d] += block[pos:pos + subs[d]]
                pos += subs[d]
        for d in range(P):
            pieces[(s, d)] = parts[d]
    out = []
    for d in range(P):
        received = b"".join(pieces[(s, d)] for s in range(P))
        old = target_slabs[d]
        out.append(received + old[len(received):])
    return out


def transpose(counts: list[list[int]]) -> list[list[int]]:
    P = len(counts)
    return [[counts[s][d] for s in range(P)] for d in range(P)]
