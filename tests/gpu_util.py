"""Shared helpers for the GPU parity tests: moving bf16 bit patterns to and from the
device, the oracle-side caches, and the GEMM tolerance of the workload definition:
|gpu - exact| <= 2^-7 |exact| + 1e-3 rms(exact), per element."""
from __future__ import annotations

import functools
import os

import numpy as np
import pytest

import workloads as W
from oracle import mx_oracle as O

TOL_REL = 2.0 ** -7
TOL_RMS = 1e-3


def torch_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def lib_or_fail():
    import mxfp4_quantized_gemm_inline_amd as mx
    if not os.path.exists(mx.LIB_PATH):
        pytest.fail("libmxgemm.so is not built: the HIP path must exist on a GPU run")
    mx.lib()
    return mx


def dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch.bfloat16).cuda()


def host_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def check_gemm(c_gpu_bits: np.ndarray, exact: np.ndarray, rms: float | None = None, what: str = ""):
    got = O.bf16_to_f64(c_gpu_bits)
    if rms is None:
        rms = float(np.sqrt(np.mean(exact * exact))) if exact.size else 0.0
    err = np.abs(got - exact)
    bound = TOL_REL * np.abs(exact) + TOL_RMS * rms
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at {tuple(i)}: "
                             f"gpu={got[tuple(i)]!r} exact={exact[tuple(i)]!r} bound={bound[tuple(i)]!r}")
    return float(err.max()) if err.size else 0.0


@functools.lru_cache(maxsize=None)
def dense_weight_cached(name: str):
    """(W bits, oracle payload, oracle scales) for a dense workload."""
    N, K, _, _ = W.DENSE_CONFIGS[name]
    w = W.dense_weight(N, K)
    qw, sw = O.quantize_mx(w)
    return w, qw, sw


@functools.lru_cache(maxsize=None)
def dense_activation_cached(name: str, M: int):
    N, K, ms, structure = W.DENSE_CONFIGS[name]
    return W.dense_activation(M, K, structure, m_max=max(max(ms), M))


def sample_rows(M: int, n: int = 48, seed: int = 0, tile: int | None = 64) -> np.ndarray:
    """All rows when M is small, else the first, the last, one seeded row inside every
    `tile`-row tile (so no row tile of any dense kernel goes unchecked: the tiled kernels use
    16-, 64-, 128- and 256-row tiles, all multiples or divisors of 64 that align with it) and
    a seeded spread of the rest, at least n rows in all. tile=None skips the per-tile rows
    (grouped outputs, whose tiles follow the expert segments and are covered by one row of
    every segment instead)."""
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    per_tile = [] if tile is None else [t0 + int(rng.integers(0, min(tile, M - t0))) for t0 in range(0, M, tile)]
    picked = set([0, M - 1] + per_tile)
    rest = np.setdiff1d(np.arange(1, M - 1), np.fromiter(picked, dtype=np.int64))
    extra = max(0, n - len(picked))
    if extra and rest.size:
        picked.update(int(r) for r in rng.choice(rest, size=min(extra, rest.size), replace=False))
    return np.array(sorted(picked))
