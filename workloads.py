"""Seeded synthetic inputs for the tests and the benchmark.

This module only draws random inputs and lays out caches; it holds none of
the quantization arithmetic, and both the GPU path and the CPU oracle are fed
from it.  Every recipe is deterministic in its seed (numpy PCG64 on the host;
torch's Philox generator on the device for the 4.5M-token case, whose host
copy the oracle reads).

Shapes and value distributions follow the workloads the store is built for:
a 512-wide post-RMSNorm MLA latent, group 32, 272-byte rows, paged caches of
64-token blocks (optionally interleaved with other layers' pages), pad slots
(-1), contiguous per-request slot runs (prefill) or scattered slots (decode).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

LATENT = 512
ROW_BYTES = 272  # 512/2 code bytes + 512/32 scale bytes
CANARY = 0xA5


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return the 16-bit patterns.
    Inputs are finite; this only shapes test data."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


@dataclass
class StoreCase:
    """One MXFP4 store workload (host arrays)."""
    name: str
    src: np.ndarray            # uint16 [T, 512] bf16 bits
    slots: np.ndarray          # int64 [T]
    num_blocks: int
    block_size: int
    block_stride_rows: int
    cache_bytes: int           # size of the whole cache buffer
    gather_slots: np.ndarray | None = None
    notes: dict = field(default_factory=dict)

    def fresh_cache(self) -> np.ndarray:
        return np.full(self.cache_bytes, CANARY, dtype=np.uint8)


# ------------------------------------------------------------------ config 0

def tiny_case(seed: int = 0) -> StoreCase:
    """64 tokens of N(0,1); flat cache of 128 slots; a permutation subset of
    slots with 8 pads at random positions."""
    rng = np.random.default_rng(seed)
    src = f32_to_bf16_bits(rng.standard_normal((64, LATENT), dtype=np.float32))
    slots = rng.permutation(128)[:64].astype(np.int64)
    slots[rng.choice(64, 8, replace=False)] = -1
    return StoreCase("tiny", src, slots, 1, 128, 128, 128 * ROW_BYTES)


# ------------------------------------------------------------------ config 1

_TIE_MULTIPLES = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float64)


def decode_case(seed: int = 1, tokens: int = 256) -> StoreCase:
    """Decode-shaped batch: Student-t(3) values times a per-row scale
    2^U(-8, 8), with injected structure per 32-value group (each with
    probability ~8%): exact powers of two (or 3 * 2^j) as the group maximum,
    exact E2M1 ties (k-anchored groups: a +-6*2^k element plus +-m*2^k for the
    midpoint multiples m), all-zero groups with mixed signed zeros, and tiny
    negatives (below a quarter of the group's scale, and exactly a quarter),
    some with extreme anchors (k = -126, -120, 20, 60, 125).  Paged cache of
    4096 blocks x 64 slots with a block stride of 192 rows (two other layers
    interleaved); distinct random slots with 10% pads."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(tokens, LATENT)) * np.exp2(rng.uniform(-8, 8, size=(tokens, 1)))
    x = x.astype(np.float64)
    groups = x.reshape(tokens, LATENT // 32, 32)
    kinds = rng.random(groups.shape[:2])
    for t in range(tokens):
        for g in range(LATENT // 32):
            grp = groups[t, g]
            r = kinds[t, g]
            if r < 0.08:  # power of two (or three times one) as the amax
                j = int(np.ceil(np.log2(np.max(np.abs(grp)) + 1e-30))) + int(rng.integers(1, 3))
                mag = 2.0 ** j * (3.0 if rng.random() < 0.5 else 1.0)
                grp[rng.integers(32)] = mag * rng.choice([-1.0, 1.0])
            elif r < 0.16:  # exact ties
                k = int(rng.integers(-10, 10))
                grp[:] = rng.choice(_TIE_MULTIPLES, 32) * rng.choice([-1.0, 1.0], 32) * 2.0 ** k
                grp[rng.integers(32)] = 6.0 * 2.0 ** k * rng.choice([-1.0, 1.0])
            elif r < 0.24:  # all-zero group, mixed signs of zero
                grp[:] = np.where(rng.random(32) < 0.5, -0.0, 0.0)
            elif r < 0.32:  # tiny negatives under a known scale
                k = int(rng.choice([-126, -120, -3, 0, 5, 20, 60, 125]))
                scale = 2.0 ** k
                grp[:] = rng.uniform(-6, 6, 32) * scale
                grp[0] = 6.0 * scale
                grp[1] = -0.25 * scale
                grp[2:10] = -rng.uniform(0, 0.25, 8) * scale
                grp[10] = -(2.0 ** (k - 140))  # tiny; still nonzero after division
                grp[11] = -0.0
                grp[12] = -(2.0 ** (k - 151))  # divided by 2^k: below half the least subnormal
                grp[13] = -(2.0 ** (k - 149))  # divided by 2^k: the least fp32 subnormal
    with np.errstate(over="ignore", under="ignore"):
        src = f32_to_bf16_bits(x.astype(np.float32))
    nb, bs, stride = 4096, 64, 192
    slots = rng.choice(nb * bs, tokens, replace=False).astype(np.int64)
    slots[rng.choice(tokens, tokens // 10, replace=False)] = -1
    return StoreCase("decode", src, slots, nb, bs, stride, nb * stride * ROW_BYTES)


# ------------------------------------------------------------------ config 2

def prefill_case(seed: int = 2, tokens: int = 16384, requests: int = 32) -> StoreCase:
    """Prefill chunk: N(0,1) times a per-row scale 2^U(-20, 20).  Paged cache
    of 8192 blocks x 64 (contiguous blocks).  32 requests with lengths
    U[448, 512), each a contiguous run of slots starting at the first slot of
    a distinct random block (runs do not overlap); the batch is padded to
    16384 tokens with -1."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, LATENT)) * np.exp2(rng.uniform(-20, 20, size=(tokens, 1)))
    src = f32_to_bf16_bits(x.astype(np.float32))
    nb, bs = 8192, 64
    lengths = rng.integers(448, 512, size=requests)
    starts = rng.choice(nb // 8, requests, replace=False) * 8  # 8 blocks = 512 slots apart
    runs = [np.arange(s * bs, s * bs + n, dtype=np.int64) for s, n in zip(starts, lengths)]
    valid = np.concatenate(runs)
    assert valid.size <= tokens
    slots = np.full(tokens, -1, dtype=np.int64)
    slots[: valid.size] = valid
    case = StoreCase("prefill", src, slots, nb, bs, bs, nb * bs * ROW_BYTES)
    case.gather_slots = valid.copy()
    return case


def request_runs_slots(tokens: int, seed: int = 2, block_size: int = 64) -> tuple[np.ndarray, int]:
    """The prefill slot pattern at any batch size: requests of U[448, 512)
    tokens, each a contiguous run of slots from the first slot of its own
    8-block (512-slot) chunk, chunks in random order, every token valid (the
    last request is cut to fit).  Returns (slots int64 [tokens], number of
    slots in the flat cache)."""
    rng = np.random.default_rng(seed)
    chunk = 8 * block_size
    lengths = rng.integers(448, 512, size=tokens // 448 + 1)
    ends = np.cumsum(lengths)
    requests = int(np.searchsorted(ends, tokens)) + 1
    lengths = lengths[:requests].copy()
    lengths[-1] -= int(ends[requests - 1]) - tokens
    starts = rng.permutation(requests).astype(np.int64) * chunk
    first = np.repeat(np.cumsum(lengths) - lengths, lengths)
    slots = np.repeat(starts, lengths) + (np.arange(tokens, dtype=np.int64) - first)
    return slots, requests * chunk


# ------------------------------------------------------------------ config 3

LARGE_TOKENS = 4_500_000


def large_case_device(tokens: int = LARGE_TOKENS, seed: int = 3, device: str = "cuda"):
    """4.5M tokens uniform in [-4, 4] (2.3e9 values, past 2^31) and a random
    permutation of the 4.5M flat slots, drawn on the device with torch's
    seeded generator.  Returns (src bf16 [T, 512], slots int64 [T])."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    src = torch.empty((tokens, LATENT), dtype=torch.bfloat16, device=device)
    # fill in chunks to bound the fp32 temporary
    chunk = 1 << 20
    for lo in range(0, tokens, chunk):
        hi = min(tokens, lo + chunk)
        tmp = torch.empty((hi - lo, LATENT), dtype=torch.float32, device=device)
        tmp.uniform_(-4.0, 4.0, generator=g)
        src[lo:hi].copy_(tmp)
        del tmp
    slots = torch.randperm(tokens, generator=g, device=device, dtype=torch.int64)
    return src, slots


def large_sample_host(tokens: int, seed: int = 3) -> tuple[np.ndarray, np.ndarray]:
    """The large workload's recipe drawn on the host (torch's CPU generator;
    same distribution as the device batch, other values), as numpy arrays
    (bf16 bits uint16 [T, 512], int64 slots), used to time the CPU oracle."""
    import torch

    src, slots = large_case_device(tokens, seed, device="cpu")
    return src.view(torch.int16).numpy().view(np.uint16), slots.numpy()


# ------------------------------------------------------------------ config 4

@dataclass
class RopeCase:
    latent: np.ndarray       # uint16 [T, 512]
    positions: np.ndarray    # int64 [T]
    cos_sin: np.ndarray      # fp32 [65536, 64]
    slots: np.ndarray        # int64 [T]
    block: int
    num_blocks: int
    compress_ratio: int


def rope_cos_sin_table(rows: int = 65536, rot_dim: int = 64, theta: float = 10000.0) -> np.ndarray:
    """GPT-J RoPE table: row p = [cos(p*w_j) for j<32 | sin(p*w_j) for j<32],
    w_j = theta^(-2j/rot_dim); built in float64, rounded once to fp32."""
    j = np.arange(rot_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * j / rot_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def rope_case(seed: int = 4, tokens: int = 16384, compress_ratio: int = 4) -> RopeCase:
    """16384 tokens of N(0,1); positions U[0, 65536); compress ratio 4;
    cache block 64 over 256 blocks; slots a random permutation of the
    16384 slots."""
    rng = np.random.default_rng(seed)
    latent = f32_to_bf16_bits(rng.standard_normal((tokens, LATENT), dtype=np.float32))
    positions = rng.integers(0, 65536, size=tokens, dtype=np.int64)
    slots = rng.permutation(tokens).astype(np.int64)
    return RopeCase(latent, positions, rope_cos_sin_table(), slots, 64, tokens // 64, compress_ratio)



ROPE_LARGE_TOKENS = 1 << 20


def rope_large_device(tokens: int = ROPE_LARGE_TOKENS, seed: int = 4, device: str = "cuda"):
    """The RoPE inserts at bandwidth scale: 1,048,576 tokens of N(0,1) bf16,
    positions U[0, 65536) into the 65536-row table of rope_case, compress
    ratio 1 (every token written), slots a random permutation of a
    [tokens / 64, 64] cache.  Drawn on the device with torch's seeded
    generator.  Returns (latent bf16 [T, 512], positions int64 [T], table
    fp32 [65536, 64], slots int64 [T])."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    table = torch.from_numpy(rope_cos_sin_table()).to(device)
    latent = torch.empty((tokens, LATENT), dtype=torch.float32, device=device).normal_(generator=g)
    latent = latent.to(torch.bfloat16)
    positions = torch.randint(0, table.shape[0], (tokens,), generator=g, device=device)
    slots = torch.randperm(tokens, generator=g, device=device)
    return latent, positions, table, slots


RING_ROWS = 262_144


def ring_large_device(rows: int = RING_ROWS, blocks: int = 8192, capacity: int = 32, width: int = 1024,
                      seed: int = 5, device: str = "cuda"):
    """The ring-state save at bandwidth scale: 262,144 fp32 rows of 1024
    values U(-1, 1) to distinct random slots of an 8192 x 32-row ring.
    Returns (rows fp32 [R, width], slots int64 [R], ring shape)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    src = torch.empty((rows, width), dtype=torch.float32, device=device).uniform_(-1.0, 1.0, generator=g)
    slots = torch.randperm(blocks * capacity, generator=g, device=device)[:rows].contiguous()
    return src, slots, (blocks, capacity, width)


def random_cache_device(rows: int, seed: int = 6, device: str = "cuda"):
    """A flat cache of `rows` 272-byte rows of uniformly random bytes (every
    code and every scale byte, 0xFF included), drawn on the device: the
    gather-dequant input at bandwidth scale.  Returns uint8 [rows * 272]."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(0, 256, (rows * ROW_BYTES,), generator=g, device=device, dtype=torch.uint8)

# ------------------------------------------------------------------ attention (read side)

@dataclass
class AttnCase:
    q: np.ndarray          # uint16 bf16 bits [T, H, 512]
    cache: np.ndarray      # uint8 [num_blocks * block_stride_rows * 272]
    num_blocks: int
    block_size: int
    block_stride_rows: int
    indices: np.ndarray    # int32 [T, topk]
    scale: float
    sink: np.ndarray | None  # fp32 [H] or None


def random_mxfp4_rows(rng: np.random.Generator, rows: int, scale_lo: int = 121,
                      scale_hi: int = 130) -> np.ndarray:
    """Random but well-formed 272-byte MXFP4 rows: uniform code bytes and
    E8M0 scale bytes uniform in [scale_lo, scale_hi] (values of order 2^-6
    .. 2^3 * 6), as uint8 [rows, 272].  Caches for the read side are drawn
    this way so that neither implementation's store produces the other's
    input."""
    out = rng.integers(0, 256, size=(rows, ROW_BYTES), dtype=np.uint8)
    out[:, 256:] = rng.integers(scale_lo, scale_hi + 1, size=(rows, 16), dtype=np.uint8)
    return out


def attention_case(tokens: int, heads: int, topk: int, seed: int, num_blocks: int = 64,
                   block_size: int = 64, block_stride_rows: int | None = None,
                   invalid_frac: float = 0.1, sink: bool = False,
                   score_std: float = 2.0) -> AttnCase:
    """Sparse-attention inputs: q ~ N(0, 1) in bf16; a paged cache of random
    well-formed rows (other layers' rows between blocks when the block
    stride exceeds the block); per token `topk` random slots of the cache
    (repeats allowed), a fraction replaced by -1 and a few by slots past the
    end; scale chosen so scores have about `score_std` standard deviation;
    optional per-head sinks ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    bsr = block_stride_rows or block_size
    rows = num_blocks * bsr
    cache = random_mxfp4_rows(rng, rows).reshape(-1)
    q = f32_to_bf16_bits(rng.standard_normal((tokens, heads, LATENT)).astype(np.float32))
    slots = num_blocks * block_size
    idx = rng.integers(0, slots, size=(tokens, topk)).astype(np.int32)
    idx[rng.random((tokens, topk)) < invalid_frac] = -1
    if topk:
        idx[rng.random((tokens, topk)) < 0.01] = slots + 7
    # a dequantized value with uniform codes (mean square 68.5/8) and a scale
    # 2^e, e uniform in [-6, 3] (mean of 4^e ~ 8.53), has rms ~ 8.55; a dot
    # product with N(0, 1) over 512 dims then has std ~ 8.55 * sqrt(512)
    scale = score_std / (8.55 * np.sqrt(LATENT))
    snk = rng.standard_normal(heads).astype(np.float32) if sink else None
    return AttnCase(q, cache, num_blocks, block_size, bsr, idx, float(scale), snk)


def attention_workload_device(tokens: int = 4096, context: int = 16384, heads: int = 32,
                              topk: int = 2048, seed: int = 5, device: str = "cuda"):
    """The read-side workload: the last `tokens` queries of a `context`-token
    prefill, each attending `topk` distinct random slots of its causal prefix
    (fewer, padded with -1, when the prefix is shorter), heads query heads,
    over a flat cache of `context` random well-formed rows.  Drawn on the
    device with torch's seeded generator.  Returns (q bf16 [T, H, 512], cache
    uint8 [context, 272], indices int32 [T, topk], scale)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    cache = torch.randint(0, 256, (context, ROW_BYTES), generator=g, device=device, dtype=torch.uint8)
    cache[:, 256:] = torch.randint(121, 131, (context, 16), generator=g, device=device, dtype=torch.uint8)
    q = torch.randn((tokens, heads, LATENT), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    pos = torch.arange(context - tokens, context, device=device)
    idx = torch.empty((tokens, topk), dtype=torch.int32, device=device)
    chunk = 512
    for lo in range(0, tokens, chunk):
        hi = min(tokens, lo + chunk)
        r = torch.rand((hi - lo, context), generator=g, device=device)
        keys = torch.arange(context, device=device)
        r[keys[None, :] > pos[lo:hi, None]] = -1.0
        val, sel = torch.topk(r, topk, dim=1)
        sel = sel.to(torch.int32)
        sel[val < 0] = -1
        idx[lo:hi] = sel
    scale = 2.0 / (8.55 * LATENT ** 0.5)   # scores of std ~2 (see attention_case)
    return q, cache, idx, scale
