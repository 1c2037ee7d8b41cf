"""Seeded synthetic workloads for the all_to_all_v exchange.

Input generation only: this module builds count matrices, payload bytes,
sentinel-filled targets and zeroed signals.  It holds none of the exchange's
arithmetic (no displacements, no placement) and imports neither the HIP
binding nor the oracle, so both sides can draw the same inputs from it.

The five workloads (c1..c5) are the exchange at growing sizes:

* c1  P=4, fp32, counts uniform in [0, 64], core_num 1 (one block).
* c2  P=8, fp32, counts uniform in [0, 4096] with 10% of entries forced to 0,
      core_num 10 (folds to 8 blocks).
* c3  P=8, int8, an MoE dispatch: 4096 tokens per source rank, each routed to
      2 distinct ranks drawn without replacement with Zipf(1.2) popularity
      (rank d has weight (d+1)^-1.2), 7168 bytes per token; core_num 64.
      The token-and-routing form follows the EP (expert parallel) data flow of
      the CANN BatchMatMulReduceScatterAllToAll page.
* c4  P=32, fp32, counts uniform in [0, 2^19] with 20% zeros, core_num 256.
* c5  P=8, fp32, equal counts 2^25: the AllToAll at the end of the CANN
      BatchMatMulReduceScatterAllToAll op, per rank (E/ep=8, ep*C=8*2048,
      H/tp=2048) to (E=64, C=2048, H/tp=2048), input already packed by
      destination; core_num 256.

Beside them, the shapes of the exchange's variants:

* c5b (:func:`bias_workload`): c5's shape in BF16 (or FP16) with the bias Add
      fused in front, nblk = E/ep = 8, rows of H/tp = 2048 elements.
* c3i (:func:`indexed_workload`): c3's MoE dispatch as the indexed exchange,
      token tables stored once and the routing as gather lists.
* c5's counts taken as the blocked exchange (nblk = 8) need no workload of
      their own: the same bytes are read as temp3's block-rows.

Payload bytes come from a counter-based SplitMix64 stream (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014; the
finalizer constants are Vigna's published splitmix64), so any byte can be
regenerated on its own: byte i of stream ``seed`` is byte ``i % 8`` (little
endian) of ``mix(seed + (i // 8 + 1) * 0x9E3779B97F4A7C15)``.  Counts and
routing come from ``numpy.random.Generator(PCG64(k))`` for workload k.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FP32 = 0
INT8 = 1
FP16 = 2
BF16 = 3
ELEM_SIZE = {FP32: 4, INT8: 1, FP16: 2, BF16: 2}
DTYPE_NAME = {FP32: "fp32", INT8: "int8", FP16: "fp16", BF16: "bf16"}
SENTINEL = 0xA5

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _signed(x: int) -> int:
    x &= (1 << 64) - 1
    return x - (1 << 64) if x >= 1 << 63 else x


# ---------------------------------------------------------------- payload bytes

def random_words_np(seed: int, first_word: int, nwords: int) -> np.ndarray:
    """SplitMix64 words ``first_word .. first_word+nwords-1`` of stream ``seed``."""
    with np.errstate(over="ignore"):
        i = np.arange(first_word + 1, first_word + 1 + nwords, dtype=np.uint64)
        z = np.uint64(seed & ((1 << 64) - 1)) + i * np.uint64(_GOLDEN)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        z = z ^ (z >> np.uint64(31))
    return z


def random_bytes_np(seed: int, start: int, n: int) -> np.ndarray:
    """Bytes ``start .. start+n-1`` of stream ``seed`` as uint8 (numpy, any offset)."""
    if n <= 0:
        return np.zeros(0, np.uint8)
    w0 = start // 8
    w1 = (start + n + 7) // 8
    b = random_words_np(seed, w0, w1 - w0).view(np.uint8)
    off = start - w0 * 8
    return b[off:off + n].copy()


def fill_random_(t, seed: int, chunk_words: int = 1 << 24) -> None:
    """Fill a flat uint8 torch tensor (CPU or GPU) with stream ``seed`` from byte 0.

    Same bits as :func:`random_bytes_np`; integer ops only, chunked so the
    temporaries stay small.  ``t.numel()`` need not be a multiple of 8.
    """
    import torch
    assert t.dtype == torch.uint8 and t.dim() == 1 and t.is_contiguous()
    n = t.numel()
    nwords = (n + 7) // 8
    g, m1, m2 = _signed(_GOLDEN), _signed(_M1), _signed(_M2)
    sd = _signed(seed)
    for w0 in range(0, nwords, chunk_words):
        w1 = min(nwords, w0 + chunk_words)
        z = torch.arange(w0 + 1, w1 + 1, dtype=torch.int64, device=t.device)
        z.mul_(g).add_(sd)
        z.bitwise_xor_((z >> 30) & ((1 << 34) - 1)).mul_(m1)
        z.bitwise_xor_((z >> 27) & ((1 << 37) - 1)).mul_(m2)
        z.bitwise_xor_((z >> 31) & ((1 << 33) - 1))
        b = z.view(torch.uint8)
        lo, hi = w0 * 8, min(n, w1 * 8)
        t[lo:hi].copy_(b[: hi - lo])


def finite16_from_words(words: np.ndarray, dtype: int) -> np.ndarray:
    """Map random 16-bit words to finite, moderate 16-bit floats (as uint16 bits).

    Random sign and mantissa; the exponent field is folded into a middle
    range (bf16: 2^-27 .. 2^27, fp16: 2^-10 .. 2^10), so no NaN, infinity or
    overflow can arise in the payload or in a sum with a moderate bias.
    """
    w = words.astype(np.uint32)
    sign = w & 0x8000
    if dtype == BF16:
        exp = 100 + (w >> 7) % 55                       # biased 100..154
        return (sign | (exp << 7) | (w & 0x7F)).astype(np.uint16)
    exp = 5 + (w >> 10) % 21                            # biased 5..25
    return (sign | (exp << 10) | (w & 0x3FF)).astype(np.uint16)


def edge16_from_words(words: np.ndarray, dtype: int) -> np.ndarray:
    """Map random 16-bit words to a mixture that reaches every IEEE class of a
    16-bit format (as uint16 bits): the top three bits pick the class, the
    rest fill sign and fraction.

    class 0-2: the word itself (any exponent, so also NaN and infinity);
    3: the largest finite magnitude; 4: the top binade (overflows when two
    such values are added); 5: +-infinity; 6: a NaN (quiet or signalling,
    random payload, all-ones fraction included); 7: zero or a subnormal.
    """
    w = words.astype(np.uint32)
    cls = w >> 13
    sign = (w << 3) & 0x8000                            # bit 12 -> sign
    frac_bits = 7 if dtype == BF16 else 10
    emax = 0xFF if dtype == BF16 else 0x1F              # all-ones exponent field
    fmask = (1 << frac_bits) - 1
    frac = w & fmask
    out = w.copy()
    out = np.where(cls == 3, sign | ((emax - 1) << frac_bits) | fmask, out)
    out = np.where(cls == 4, sign | ((emax - 1) << frac_bits) | frac, out)
    out = np.where(cls == 5, sign | (emax << frac_bits), out)
    out = np.where(cls == 6, sign | (emax << frac_bits) | np.maximum(frac, 1), out)
    out = np.where(cls == 7, sign | (frac & (fmask >> (w >> 11 & 1))), out)
    return out.astype(np.uint16)


def edge_bias_values(seed: int, P: int, nblk: int, hidden: int, dtype: int) -> np.ndarray:
    """Bias [P, nblk, hidden] reaching every IEEE class: float32 for BF16
    payloads (random bit patterns, the largest finite values, infinities,
    NaNs, subnormals, moderate values), binary16 bits from
    :func:`edge16_from_words` for FP16."""
    n = P * nblk * hidden
    if dtype == BF16:
        u = random_bytes_np(seed, 0, 4 * n).view(np.uint32)
        cls = u & 7
        sign = u & 0x80000000
        out = u.copy()                                   # class 0-1: any pattern
        out = np.where(cls == 2, sign | 0x7F7FFFFF, out)                 # largest finite
        out = np.where(cls == 3, sign | 0x7F000000 | (u >> 9 & 0x7FFFFF), out)  # top binades
        out = np.where(cls == 4, sign | 0x7F800000, out)                 # infinity
        out = np.where(cls == 5, sign | 0x7F800000 | np.maximum(u >> 9 & 0x7FFFFF, 1), out)  # NaN
        out = np.where(cls == 6, sign | (u >> 9 & 0x7FFFFF), out)        # zero or subnormal
        out = np.where(cls == 7, sign | 0x3F800000 | (u >> 9 & 0x7FFFFF), out)  # [1, 2)
        return out.astype(np.uint32).view(np.float32).reshape(P, nblk, hidden)
    w = random_bytes_np(seed, 0, 2 * n).view(np.uint16)
    return edge16_from_words(w, FP16).reshape(P, nblk, hidden)


def finite16_(t, dtype: int, chunk: int = 1 << 26) -> None:
    """In place on a torch tensor of 16-bit words (any 2-byte dtype, CPU or GPU):
    the same mapping as :func:`finite16_from_words`, integer ops only."""
    import torch
    v = t.view(torch.int16).view(-1)
    for i in range(0, v.numel(), chunk):
        w = v[i:i + chunk].to(torch.int32) & 0xFFFF
        sign = w & 0x8000
        if dtype == BF16:
            out = sign | ((100 + (w >> 7) % 55) << 7) | (w & 0x7F)
        else:
            out = sign | ((5 + (w >> 10) % 21) << 10) | (w & 0x3FF)
        out -= (out >> 15) << 16                        # to the int16 range
        v[i:i + chunk] = out.to(torch.int16)


def bias_values(seed: int, P: int, nblk: int, hidden: int, dtype: int) -> np.ndarray:
    """Bias [P, nblk, hidden]: float32 for BF16 payloads, binary16 bits for FP16."""
    n = P * nblk * hidden
    if dtype == BF16:
        u = random_bytes_np(seed, 0, 4 * n).view(np.uint32)
        v = ((u >> 9).astype(np.float64) / float(1 << 23) - 0.5) * 64.0   # in [-32, 32)
        return v.astype(np.float32).reshape(P, nblk, hidden)
    w = random_bytes_np(seed, 0, 2 * n).view(np.uint16)
    return finite16_from_words(w, FP16).reshape(P, nblk, hidden)


# ---------------------------------------------------------------- count matrices

def uniform_counts(rng: np.random.Generator, P: int, hi: int, zero_frac: float) -> np.ndarray:
    """Counts uniform in [0, hi] with exactly round(zero_frac*P*P) entries forced to 0."""
    C = rng.integers(0, hi + 1, size=(P, P), dtype=np.int64)
    nz = int(round(zero_frac * P * P))
    if nz:
        idx = rng.choice(P * P, size=nz, replace=False)
        C.reshape(-1)[idx] = 0
    return C.astype(np.int32)


def moe_routing(rng: np.random.Generator, P: int, tokens: int, topk: int,
                zipf_s: float) -> np.ndarray:
    """bool [P(src), tokens, P(dst)]: each token picks ``topk`` distinct ranks.

    Sampling without replacement proportional to weight (d+1)^-s, done with
    the Gumbel-top-k construction (equivalent to drawing ranks one at a time
    without replacement, each draw proportional to the remaining weights).
    """
    logw = -zipf_s * np.log(np.arange(1, P + 1, dtype=np.float64))
    keys = logw[None, None, :] + rng.gumbel(size=(P, tokens, P))
    top = np.argsort(-keys, axis=2, kind="stable")[:, :, :topk]
    mask = np.zeros((P, tokens, P), dtype=bool)
    np.put_along_axis(mask, top, True, axis=2)
    return mask


# ---------------------------------------------------------------- workloads

@dataclass
class Workload:
    name: str
    description: str
    P: int
    dtype: int
    core_num: int
    S: int
    in_slab: int            # bytes per input slab
    tgt_slab: int           # bytes per target slab
    counts: np.ndarray      # int32 [P, P], elements
    payload_seed: int
    # c3 only: token payloads are duplicated into both destinations.
    routing: np.ndarray | None = None
    token_bytes: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def elem(self) -> int:
        return ELEM_SIZE[self.dtype]

    @property
    def payload_bytes(self) -> int:
        return int(self.counts.astype(np.int64).sum()) * self.elem

    @property
    def in_bytes(self) -> int:
        return self.P * self.in_slab

    @property
    def tgt_bytes(self) -> int:
        return self.P * self.tgt_slab

    def summary(self) -> dict:
        return {"workload": self.name, "P": self.P,
                "dtype": DTYPE_NAME[self.dtype],
                "core_num": self.core_num, "signal": [self.P, self.S],
                "in_slab_bytes": self.in_slab, "tgt_slab_bytes": self.tgt_slab,
                "payload_bytes": self.payload_bytes}


def workload(k: int, scale: int = 1) -> Workload:
    """Workload c``k`` (k = 1..5).  ``scale`` > 1 shrinks c3..c5 for quick tests
    (the count distribution keeps its shape, sizes divide by ``scale``)."""
    rng = np.random.Generator(np.random.PCG64(k))
    seed = 1000 + k
    if k == 1:
        P = 4
        C = uniform_counts(rng, P, 64, 0.0)
        slab = 64 * P * 4
        return Workload("c1_p4_fp32_uniform64", "P=4 fp32 counts U[0,64], core_num 1",
                        P, FP32, 1, 1, slab, slab, C, seed)
    if k == 2:
        P = 8
        C = uniform_counts(rng, P, 4096, 0.1)
        slab = 4096 * P * 4
        return Workload("c2_p8_fp32_uniform4096", "P=8 fp32 counts U[0,4096] 10% zero, core_num 10",
                        P, FP32, 10, 8, slab, slab, C, seed)
    if k == 3:
        P, tokens, hidden = 8, 4096 // scale, 7168
        route = moe_routing(rng, P, tokens, 2, 1.2)
        n = route.sum(axis=1).astype(np.int64)          # [src, dst] tokens
        C = (n * hidden).astype(np.int32)
        return Workload("c3_p8_int8_moe_top2_zipf1.2", "P=8 int8 MoE dispatch, 4096 tok/rank top-2 "
                        "Zipf(1.2), hidden 7168, core_num 64",
                        P, INT8, 64, 64, 2 * tokens * hidden, P * tokens * hidden, C, seed,
                        routing=route, token_bytes=hidden)
    if k == 4:
        P = 32
        hi = (1 << 19) // scale
        C = uniform_counts(rng, P, hi, 0.2)
        slab = P * hi * 4
        return Workload("c4_p32_fp32_uniform2^19", "P=32 fp32 counts U[0,2^19] 20% zero, core_num 256",
                        P, FP32, 256, 256, slab, slab, C, seed)
    if k == 5:
        P = 8
        n = (1 << 25) // scale                          # (E/ep)*C*(H/tp) elements
        C = np.full((P, P), n, dtype=np.int32)
        slab = P * n * 4
        return Workload("c5_p8_fp32_equal_bmm_rs_a2a", "P=8 fp32 equal counts 2^25 "
                        "(E/ep=8, ep*C=8*2048, H/tp=2048) -> (E=64, C=2048, H/tp=2048), core_num 256",
                        P, FP32, 256, 256, slab, slab, C, seed,
                        extra={"E_over_ep": 8, "ep": 8, "C": 2048 // scale, "H_over_tp": 2048})
    raise ValueError(f"no workload c{k}")


def bias_workload(dtype: int = BF16, scale: int = 1) -> Workload:
    """c5's exchange in 16 bits with the bias Add fused in front: the tail of the
    CANN BatchMatMulReduceScatterAllToAll op with a BF16 (or FP16) x, per rank
    temp2 (E/ep=8, ep*C=8*2048, H/tp=2048) plus bias (E/ep, 1, H/tp), then the
    AllToAll; nblk = E/ep = 8, rows of H/tp = 2048 elements, core_num 256.
    The payload is finite 16-bit floats (:func:`input16_np`); the bias comes
    from :func:`bias_values` with seed ``payload_seed + 1``."""
    P, A, H = 8, 8, 2048
    n = (1 << 25) // scale
    C = np.full((P, P), n, dtype=np.int32)
    slab = P * n * 2
    tag = "bf16_fp32bias" if dtype == BF16 else "fp16_fp16bias"
    key = "c5b" if dtype == BF16 else "c5h"
    return Workload(f"{key}_p8_{tag}_bmm_rs_a2a", f"P=8 {tag} equal counts 2^25, bias Add fused, "
                    "(E/ep=8, ep*C=8*2048, H/tp=2048) -> (E=64, C=2048, H/tp=2048), core_num 256",
                    P, dtype, 256, 256, slab, slab, C, 1005,
                    extra={"E_over_ep": A, "ep": 8, "C": 2048 // scale, "H_over_tp": H,
                           "nblk": A, "hidden": H})


def indexed_workload(scale: int = 1) -> Workload:
    """c3's MoE dispatch taken as the indexed exchange: input slab s is source
    s's token table (tokens x 7168 int8 rows, every token stored once) and the
    gather list index[s] names, for d = 0..P-1 in turn, the tokens routed to d
    in ascending token order.  Same routing, counts, core_num and payload
    stream as c3, so the token table of source s is byte for byte the ``tok``
    block c3 packs from; ``extra`` holds the int32 [P, 2*tokens] index, the
    row length and the index stride (every token goes to exactly 2 ranks)."""
    w3 = workload(3, scale)
    P, tokens, H = w3.P, w3.routing.shape[1], w3.token_bytes
    index = np.zeros((P, 2 * tokens), np.int32)
    for s in range(P):
        k = 0
        for d in range(P):
            t = np.nonzero(w3.routing[s, :, d])[0]
            index[s, k:k + t.size] = t
            k += t.size
        assert k == 2 * tokens
    return Workload("c3i_p8_int8_moe_top2_zipf1.2_indexed",
                    "P=8 int8 MoE dispatch as a row gather: token tables of 4096 x 7168, "
                    "top-2 Zipf(1.2) routing as the index, core_num 64",
                    P, INT8, w3.core_num, w3.S, tokens * H, w3.tgt_slab, w3.counts.copy(),
                    w3.payload_seed,
                    extra={"index": index, "row_elems": H, "index_stride": 2 * tokens})


def custom(P: int, dtype: int, counts: np.ndarray, core_num: int = 1, S: int | None = None,
           in_slab: int | None = None, tgt_slab: int | None = None, seed: int = 7,
           name: str = "custom") -> Workload:
    """A workload with the given counts; slabs default to the exact maxima (rounded to 16)."""
    C = np.ascontiguousarray(counts, dtype=np.int32)
    e = ELEM_SIZE[dtype]
    rows = int(C.astype(np.int64).sum(axis=1).max(initial=0)) * e
    cols = int(C.astype(np.int64).sum(axis=0).max(initial=0)) * e
    if in_slab is None:
        in_slab = max(16, (rows + 15) // 16 * 16)
    if tgt_slab is None:
        tgt_slab = max(16, (cols + 15) // 16 * 16)
    if S is None:
        S = max(1, core_num if core_num < P else (core_num // P) * P)
    return Workload(name, name, P, dtype, core_num, S, in_slab, tgt_slab, C, seed)


# ---------------------------------------------------------------- buffers

def input_bytes_np(w: Workload) -> np.ndarray:
    """The whole input allocation as uint8 numpy (host)."""
    if w.routing is None:
        return random_bytes_np(w.payload_seed, 0, w.in_bytes)
    return _moe_input(w, np)


def input16_np(w: Workload) -> np.ndarray:
    """Input allocation of finite 16-bit floats (FP16/BF16 workloads), uint8 view."""
    words = random_bytes_np(w.payload_seed, 0, w.in_bytes).view(np.uint16)
    return finite16_from_words(words, w.dtype).view(np.uint8)


def input16_tensor(w: Workload, device):
    """:func:`input16_np` built on ``device`` (flat uint8 torch tensor)."""
    t = input_tensor(w, device)
    finite16_(t, w.dtype)
    return t


def bias_np(w: Workload, nblk: int, hidden: int) -> np.ndarray:
    return bias_values(w.payload_seed + 1, w.P, nblk, hidden, w.dtype)


def bias_tensor(w: Workload, nblk: int, hidden: int, device):
    """The bias as the torch dtype the library takes: float32 for BF16 payloads,
    float16 for FP16."""
    import torch
    b = bias_np(w, nblk, hidden)
    if w.dtype == FP16:
        return torch.from_numpy(b.view(np.float16).copy()).to(device)
    return torch.from_numpy(b).to(device)


def input_tensor(w: Workload, device):
    """The whole input allocation as a flat uint8 torch tensor on ``device``."""
    import torch
    t = torch.empty(w.in_bytes, dtype=torch.uint8, device=device)
    if w.routing is None:
        fill_random_(t, w.payload_seed)
        return t
    tok = torch.empty(w.P * w.routing.shape[1] * w.token_bytes, dtype=torch.uint8, device=device)
    fill_random_(tok, w.payload_seed)
    tok = tok.view(w.P, w.routing.shape[1], w.token_bytes)
    slabs = t.view(w.P, w.in_slab)
    for s in range(w.P):
        pos = 0
        for d in range(w.P):
            idx = np.nonzero(w.routing[s, :, d])[0]
            n = idx.size * w.token_bytes
            if n:
                src = tok[s].index_select(0, torch.as_tensor(idx, device=device))
                slabs[s, pos:pos + n].copy_(src.reshape(-1))
            pos += n
        if pos < w.in_slab:
            slabs[s, pos:].fill_(0)
    return t


def _moe_input(w: Workload, xp) -> np.ndarray:
    tokens = w.routing.shape[1]
    tok = random_bytes_np(w.payload_seed, 0, w.P * tokens * w.token_bytes)
    tok = tok.reshape(w.P, tokens, w.token_bytes)
    out = np.zeros((w.P, w.in_slab), np.uint8)
    for s in range(w.P):
        pos = 0
        for d in range(w.P):
            idx = np.nonzero(w.routing[s, :, d])[0]
            n = idx.size * w.token_bytes
            out[s, pos:pos + n] = tok[s, idx].reshape(-1)
            pos += n
    return out.reshape(-1)


def target_np(w: Workload) -> np.ndarray:
    return np.full(w.tgt_bytes, SENTINEL, np.uint8)


def signal_np(w: Workload) -> np.ndarray:
    return np.zeros((w.P, w.S), np.int32)
