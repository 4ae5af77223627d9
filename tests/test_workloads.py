"""The seeded input generators: shapes, structure and prefix property."""
import math

import numpy as np

import workloads as W


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, -0.0], dtype=np.float32)
    b = W.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6... mantissa 2)
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000, 0x8000]


def test_prefix_property():
    a_big = W.dense_activation(64, 768, "outlier_channels", m_max=2048)
    a_small = W.dense_activation(3, 768, "outlier_channels", m_max=2048)
    assert np.array_equal(a_big[:3], a_small)


def test_outlier_channels():
    K = 768
    a = W.bf16_bits_to_f32(W.dense_activation(2048, K, "outlier_channels"))
    col_std = a.std(axis=0)
    big = np.flatnonzero(col_std > 5)
    assert big.size == round(0.01 * K)


def test_zero_blocks_structure():
    M, K = 2048, 7168
    a = W.dense_activation(M, K, "zero_blocks")
    blocks = a.reshape(M, K // 32, 32)
    zero = np.all((blocks & 0x7FFF) == 0, axis=-1)
    rows = np.flatnonzero(zero.any(axis=1))
    assert rows.size == math.ceil(0.005 * M) and rows[0] == 0
    for r in rows:
        first = np.flatnonzero(zero[r])[0]
        assert np.all(blocks[r, first] == 0x8000)
    # M = 1 still carries a zero block
    a1 = W.dense_activation(1, K, "zero_blocks", m_max=2048)
    assert np.all((a1.reshape(K // 32, 32) & 0x7FFF) == 0, axis=-1).any()


def test_moe_routing():
    T = 16
    ids, offs, row_token = W.moe_routing(T)
    assert ids.shape == (T, 16)
    for t in range(T):
        assert len(set(ids[t].tolist())) == 16
    assert offs[0] == 0 and offs[-1] == T * 16 and np.all(np.diff(offs) >= 0)
    for e in range(W.MOE_E):
        toks = row_token[offs[e]:offs[e + 1]]
        assert np.all(np.diff(toks) > 0)
        for t in toks:
            assert e in ids[t]


def test_expert_weight_rows_are_a_prefix():
    """The per-expert row prefix used by the layer-shape parity tests equals the first rows
    of the full expert weight, for GEMM1 and GEMM2 seeds."""
    for e in (0, 7, 895):
        full = W.moe_expert_weight(e)
        assert np.array_equal(W.moe_expert_weight_rows(e, 64), full[:64])
        full2 = W.moe_expert_weight2(e)
        assert np.array_equal(W.moe_expert_weight_rows(e, 32, K=W.MOE_K2, seed_base=W.SEED_EXPERT2_BASE),
                              full2[:32])
