"""Seeded synthetic inputs for the dense and grouped A4W4 MXFP4 GEMM workloads.

This module is the only code shared by the CPU oracle side (tests, the bench's
CPU baseline) and the GPU side. It holds no MXFP4 arithmetic: it draws numbers,
rounds them once to bfloat16 and lays them out. Every tensor is returned as raw
bfloat16 bit patterns (numpy ``uint16``) so both sides start from the same bits.

Recipes (the shapes are those of the microbenchmark table in "[gfx950][FlyDSL]
Add direct dense A4W4 MXFP4 GEMM", section "Kernel microbenchmark", and the
grouped shape of "[gfx1250] Fuse A4W4 stage1 FP4 quantization", section
"Performance"; the value distributions are stated by the workload definitions):

* RNG: numpy PCG64 (``default_rng``). A uses seed 0, W seed 1, structure
  (outlier channels, zero blocks) seed 2, routing seed 3, expert e's W seed
  1000 + e.
* Values: float32 standard normals, scaled, then rounded once to bfloat16 with
  round-to-nearest-even.
* A is drawn once at the largest M of a sweep and smaller M take its leading
  rows, so an M-prefix of the input is the input at smaller M.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_A = 0
SEED_W = 1
SEED_STRUCT = 2
SEED_ROUTE = 3
SEED_EXPERT_BASE = 1000

W_STD = 0.02
M_SWEEP = (1, 8, 32, 128, 512, 2048)
M_TAILS = (3, 17, 100)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite. NaN is never produced by the generators here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, seed: int, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


# --------------------------------------------------------------------------- dense

DENSE_CONFIGS = {
    # name: (N, K, M list, A structure)
    "smoke_16x256x256": (256, 256, (16,), "plain"),
    "n7168_k768": (7168, 768, M_SWEEP, "outlier_channels"),
    "n7168_k4224": (7168, 4224, M_SWEEP + M_TAILS, "plain"),
    "n1536_k7168": (1536, 7168, M_SWEEP, "zero_blocks"),
    "n8448_k7168": (8448, 7168, M_SWEEP, "zero_blocks"),
}


def dense_weight(N: int, K: int, seed: int = SEED_W) -> np.ndarray:
    """W [N, K] bf16 bits, ~N(0, 0.02)."""
    return normal_bf16((N, K), seed, W_STD)


def dense_activation(M: int, K: int, structure: str = "plain", m_max: int | None = None,
                     seed: int = SEED_A) -> np.ndarray:
    """A [M, K] bf16 bits, ~N(0, 1), with the structure of the workload.

    ``outlier_channels``: round(0.01 K) channels, chosen without replacement
    (structure seed), are multiplied by 20 before the bfloat16 rounding.
    ``zero_blocks``: ceil(0.005 M_max) rows (at least one) chosen from the first
    M_max rows; in each, every 32-element block is zeroed with probability 1/4
    (at least one block per row), and the first zeroed block of each row is
    written as negative zero.
    The draw is made at ``m_max`` rows (default ``M``) and the first M rows are
    returned, so prefixes agree across a sweep.
    """
    m_max = max(M, m_max or M)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(m_max * K, dtype=np.float32).reshape(m_max, K)
    if structure == "outlier_channels":
        srng = np.random.default_rng(SEED_STRUCT)
        n_out = int(round(0.01 * K))
        ch = srng.choice(K, size=n_out, replace=False)
        x[:, ch] *= np.float32(20.0)
        bits = f32_to_bf16_bits(x)
    elif structure == "zero_blocks":
        bits = f32_to_bf16_bits(x)
        srng = np.random.default_rng(SEED_STRUCT)
        n_rows = max(1, math.ceil(0.005 * m_max))
        # row 0 is always one of them so that every prefix (M >= 1) has one
        rest = srng.choice(np.arange(1, m_max), size=n_rows - 1, replace=False) if n_rows > 1 else []
        rows = np.concatenate([[0], np.sort(np.asarray(rest, dtype=np.int64))]).astype(np.int64)
        nb = K // 32
        for r in rows:
            z = srng.random(nb) < 0.25
            if not z.any():
                z[srng.integers(nb)] = True
            blocks = np.flatnonzero(z)
            for j, b in enumerate(blocks):
                bits[r, 32 * b:32 * (b + 1)] = 0x8000 if j == 0 else 0x0000
    elif structure == "plain":
        bits = f32_to_bf16_bits(x)
    else:
        raise ValueError(f"unknown structure {structure!r}")
    return np.ascontiguousarray(bits[:M])


def dense_case(name: str, M: int):
    """(A bits [M,K], W bits [N,K], N, K) for one point of a dense workload."""
    N, K, ms, structure = DENSE_CONFIGS[name]
    A = dense_activation(M, K, structure, m_max=max(max(ms), M))
    W = dense_weight(N, K)
    return A, W, N, K


# --------------------------------------------------------------------------- grouped MoE

MOE_E = 896
MOE_TOPK = 16
MOE_K = 3584      # model_dim
MOE_N = 1536      # gate + up = 2 * inter_dim (768)
MOE_TOKENS = (1, 16, 256, 4096)


def moe_routing(T: int, E: int = MOE_E, topk: int = MOE_TOPK, seed: int = SEED_ROUTE):
    """Uniform top-k routing: every token picks ``topk`` distinct experts.

    Returns (topk_ids [T, topk] int32, expert_offsets [E+1] int32,
    row_token [T*topk] int32). Rows are sorted by expert (stable in token
    order); row r of the grouped output belongs to token row_token[r] and to
    the expert e with expert_offsets[e] <= r < expert_offsets[e+1].
    """
    rng = np.random.default_rng(seed)
    ids = np.empty((T, topk), dtype=np.int32)
    for t in range(T):
        ids[t] = rng.choice(E, size=topk, replace=False)
    flat_e = ids.reshape(-1)
    flat_t = np.repeat(np.arange(T, dtype=np.int32), topk)
    order = np.argsort(flat_e, kind="stable")
    row_token = flat_t[order].astype(np.int32)
    counts = np.bincount(flat_e, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return ids, offsets, row_token


def moe_activation(T: int, K: int = MOE_K) -> np.ndarray:
    return dense_activation(T, K, "plain", m_max=max(MOE_TOKENS + (T,)))


def moe_expert_weight(e: int, N: int = MOE_N, K: int = MOE_K) -> np.ndarray:
    return normal_bf16((N, K), SEED_EXPERT_BASE + e, W_STD)


def moe_expert_weight_rows(e: int, rows: int, K: int = MOE_K, seed_base: int = SEED_EXPERT_BASE) -> np.ndarray:
    """The first ``rows`` rows of an expert weight (GEMM1 by default; seed_base =
    SEED_EXPERT2_BASE with K = MOE_K2 for GEMM2), drawn without the rest: the draws are
    sequential in row-major order, so this is exactly a prefix of the full matrix."""
    return normal_bf16((rows, K), seed_base + e, W_STD)


# GEMM2 (down projection) of the same layer: h [rows, inter_dim] x W2_e [model_dim, inter_dim]
MOE_N2 = 3584     # model_dim
MOE_K2 = 768      # inter_dim
SEED_EXPERT2_BASE = 2000
SEED_COMBINE = 4


def moe_expert_weight2(e: int, N: int = MOE_N2, K: int = MOE_K2) -> np.ndarray:
    """W2_e [N, K] bf16 bits, ~N(0, 0.02)."""
    return normal_bf16((N, K), SEED_EXPERT2_BASE + e, W_STD)


def moe_token_rows(ids: np.ndarray) -> np.ndarray:
    """[T, topk] int32: the expert-sorted row of token t's k-th expert (the inverse of the
    stable sort moe_routing applies)."""
    T, topk = ids.shape
    order = np.argsort(ids.reshape(-1), kind="stable")
    pos = np.empty_like(order)
    pos[order] = np.arange(order.size)
    return pos.reshape(T, topk).astype(np.int32)


def moe_combine_weights(T: int, topk: int = MOE_TOPK, seed: int = SEED_COMBINE) -> np.ndarray:
    """[T, topk] float32 routing weights: a softmax of standard-normal logits per token."""
    z = np.random.default_rng(seed).standard_normal((T, topk)).astype(np.float32)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def mx_bytes(R: int, K: int, seed: int, scale_lo: int = 118, scale_hi: int = 130):
    """Arbitrary MXFP4 rows in canonical form: uniform payload bytes [R, K/2] (every E2M1
    code, both signs) and E8M0 scale bytes [R, K/32] uniform in [scale_lo, scale_hi)."""
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 256, size=(R, K // 2), dtype=np.uint8),
            rng.integers(scale_lo, scale_hi, size=(R, K // 32), dtype=np.uint8))


def moe_expert_weights(experts, N: int = MOE_N, K: int = MOE_K, threads: int = 8):
    """Yield (e, W_e bits) for the given experts, generated on a thread pool.

    Work is submitted in small batches so at most about 2 * threads expert
    matrices are held at once.
    """
    experts = list(experts)
    step = max(1, 2 * threads)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        for i in range(0, len(experts), step):
            chunk = experts[i:i + step]
            for e, w in zip(chunk, ex.map(lambda e: moe_expert_weight(e, N, K), chunk)):
                yield e, w
