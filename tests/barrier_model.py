"""An event model of the exchange's block barrier, written apart from the
oracle: it pins the oracle's signal update against the protocol it stands for.

What the pages fix about the signal:
- it is an [NR, S] int32 array with S >= B, and every admitted block takes
  part in a block-aware barrier whose blocks are all resident at once; a
  start that cannot admit them all is refused, never half-run (PyPTO
  "LowerL2TensorCollectives Pass" page, "Launch width");
- reusing the same signal array orders one exchange after the other (same
  page, "A5 URMA indexed exchange");
- the start barrier of the "vccl alltoallv dev log" page (section 6.1) gives
  each peer a sequence counter: a peer bumps its own counter by one, and the
  others wait until they see it one past the value it had when the barrier
  began.

The model takes those rules literally.  The participants of one exchange are
the admitted blocks (r, b), r < P, b < B.  Participant (r, b) owns counter
(r, b), an unsigned 32-bit value that wraps.  In one exchange each
participant reads the common entry value, posts once (its counter + 1), and
then waits until every participant's counter has moved past the entry value,
compared wrap-safely (the signed 32-bit difference is at least one).  The
participants advance one step at a time in a random interleaving, so a wait
may be polled many times before it passes; the model asserts that no wait
passes before every participant has posted, and that every wait ends.
Counters of entries that are not participants are never touched.  An
exchange whose participants do not all start from one value is refused
(some wait could never end, or would end early) and changes nothing; so is
one with B > S (a participant without a counter).

Nothing here reads or calls the oracle or the GPU library.
"""
from __future__ import annotations

import numpy as np

_MASK = 0xFFFFFFFF


def _signed32(v: int) -> int:
    v &= _MASK
    return v - (1 << 32) if v >= (1 << 31) else v


class BarrierModel:
    def __init__(self, signal: np.ndarray):
        P, S = signal.shape
        self.P, self.S = P, S
        self.counter = {(r, c): int(signal[r, c]) & _MASK for r in range(P) for c in range(S)}

    def exchange(self, B: int, rng: np.random.Generator) -> bool:
        """One exchange with B admitted blocks; False if it is refused."""
        if B < 1 or B > self.S:
            return False
        parts = [(r, b) for r in range(self.P) for b in range(B)]
        entry = {p: self.counter[p] for p in parts}
        if len(set(entry.values())) != 1:
            return False
        e0 = entry[parts[0]]
        state = dict.fromkeys(parts, "post")
        pending = list(parts)
        while pending:
            k = int(rng.integers(len(pending)))
            p = pending[k]
            if state[p] == "post":
                self.counter[p] = (self.counter[p] + 1) & _MASK
                state[p] = "wait"
                continue
            # A poll: has every participant moved one past the entry value?
            if all(_signed32(self.counter[q] - e0) >= 1 for q in parts):
                assert all(state[q] != "post" for q in parts), "a wait passed before all posts"
                state[p] = "done"
                pending[k] = pending[-1]
                pending.pop()
        assert all(_signed32(self.counter[q] - e0) == 1 for q in parts)
        return True

    def signal(self) -> np.ndarray:
        out = np.empty((self.P, self.S), np.int64)
        for (r, c), v in self.counter.items():
            out[r, c] = _signed32(v)
        return out.astype(np.int32)
