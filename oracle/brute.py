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


def transpose(counts: list[list[int]]) -> list[list[int]]:
    P = len(counts)
    return [[counts[s][d] for s in range(P)] for d in range(P)]
