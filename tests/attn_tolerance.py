"""Parity tolerance for sparse_mla_attention against the oracle's
double-precision attention over the bf16 dequantized cache, derived from
the kernel's arithmetic (used by the GPU parity tests and checked on the CPU
against an emulation of the kernel's roundings).

Scores: bf16 x bf16
products are exact in fp32 and the MFMAs accumulate 512 of them in fp32, so
|dS_j| <= g * |scale| * sum_d |q_d v_jd| with g = 2^-18 (a generous bound on
32 chained fp32 accumulations); a score error e moves each softmax weight by
a relative e - e_max, so the output moves by at most 4 g * SQ * A, with
SQ = max_j |scale| * sum_d |q_d v_jd| and A_d = sum_j p_j |v_jd| / Z (p the
exact weights, Z their sum with the sink term).  The base-2 exponent
(scale * log2 e rounded to fp32, exp2 in fp32) adds at most
2^-19 * (1 + max|s|) relative per weight.  The weights are rounded to bf16
for the weighted sum (relative 2^-9 each: at most 2^-9 * A) while the
denominator uses the fp32 weights (at most 2^-9 * |out|), and the result is
rounded to bf16 (2^-9 * |out|).  Below the fp32 normal range those
relative bounds give way to absolute ones: the hardware exp2 flushes
results under 2^-126 to zero, which drops a weight (at most 2^8 relative to
the running maximum, as that moves only past a slack of 8) or, in the split
form's merge, a key range's factor, an error under 2^-118 per listed key
against a weight sum of at least 1; and a bf16 result under 2^-126 is
rounded to a step of 2^-133.  Hence, per element, with a factor of two to
spare on the relative terms,
  |gpu - exact| <= (2^-8 + 4 g SQ + 2^-19 (1 + max|s|)) * A + 2^-7 * |exact|
                   + 2^-118 * sum_j |v_jd| + 2^-133.
"""

import numpy as np

import oracle

G = 2.0 ** -18


def dequant_rows(cache: np.ndarray, nb: int, bs: int, bsr: int, slots: np.ndarray) -> np.ndarray:
    """Rows of the listed slots as float64 (the oracle's pinned dequant);
    invalid slots give zero rows (they carry no weight anyway)."""
    flat = np.asarray(slots, dtype=np.int64).reshape(-1)
    out = np.zeros((flat.size, 512), dtype=np.uint16)
    good = (flat >= 0) & (flat < nb * bs)
    if good.any():
        out[good] = oracle.mxfp4_gather_dequant(cache, nb, bs, bsr, 512, flat[good])
    return (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(*np.shape(slots), 512)


def tolerance(q_bits, cache, nb, bs, bsr, idx, scale, sink, exact):
    qd = (q_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)   # [T, H, D]
    tol = np.zeros_like(exact)
    for t in range(idx.shape[0]):
        good = (idx[t] >= 0) & (idx[t] < nb * bs)
        if not good.any():
            continue
        v = dequant_rows(cache, nb, bs, bsr, idx[t][good])                      # [J, D]
        s = scale * (qd[t] @ v.T)                                                # [H, J]
        sq = abs(scale) * (np.abs(qd[t]) @ np.abs(v).T).max(axis=1)              # [H]
        m = s.max(axis=1)
        if sink is not None:
            m = np.maximum(m, sink.astype(np.float64))
        p = np.exp(s - m[:, None])
        z = p.sum(axis=1) + (np.exp(sink.astype(np.float64) - m) if sink is not None else 0.0)
        a = (p @ np.abs(v)) / z[:, None]                                         # [H, D]
        rel = 2.0 ** -8 + 4 * G * sq + 2.0 ** -19 * (1.0 + np.abs(s).max(axis=1))
        tol[t] = rel[:, None] * a + 2.0 ** -7 * np.abs(exact[t]) + 2.0 ** -118 * np.abs(v).sum(axis=0)[None, :] + 2.0 ** -133
    return tol
