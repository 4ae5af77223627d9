"""Pins of the second-GEMM and combine oracle functions (oracle/mx_oracle.py) to facts
outside themselves: the grouped GEMM on MXFP4 rows reduces to the (separately pinned) GEMM1
oracle when its rows are the quantized routed activations; the combine equals a brute-force
loop, selects a row under one-hot weights and ignores out-of-range rows; the token-to-row
map inverts the routing's sort."""
import numpy as np

import workloads as W
from oracle import mx_oracle as O


def test_grouped_mx_reduces_to_gemm1_oracle():
    K, N, E, T = 128, 64, 3, 6
    a = W.dense_activation(T, K, "plain", seed=11)
    ws = {e: W.dense_weight(N, K, seed=110 + e) for e in range(E)}
    offs = np.array([0, 3, 3, 7], dtype=np.int32)
    row_token = np.array([5, 0, 2, 1, 4, 3, 0], dtype=np.int32)
    qa, sa = O.quantize_mx(a[row_token])
    y = O.grouped_gemm_mx_ref(qa, sa, offs, lambda e: ws[e])
    assert np.array_equal(y, O.grouped_gemm_ref(a, row_token, offs, lambda e: ws[e]))
    rows = np.array([6, 0, 4])
    assert np.array_equal(O.grouped_gemm_mx_ref(qa, sa, offs, lambda e: ws[e], rows=rows), y[rows])


def test_combine_brute_force_one_hot_and_range():
    rng = np.random.default_rng(12)
    y = rng.normal(size=(9, 5))
    tr = np.array([[0, 4, 8], [2, 2, 7], [-1, 3, 9]], dtype=np.int32)     # -1 and 9 are out of range
    w = rng.random((3, 3)).astype(np.float32)
    out = O.combine_ref(y, tr, w)
    want = np.zeros((3, 5))
    for t in range(3):
        for k in range(3):
            if 0 <= tr[t, k] < 9:
                for n in range(5):
                    want[t, n] += float(w[t, k]) * y[tr[t, k], n]
    assert np.allclose(out, want, rtol=1e-15, atol=0)
    onehot = np.zeros((3, 3), dtype=np.float32)
    onehot[:, 1] = 1.0
    assert np.array_equal(O.combine_ref(y, tr, onehot), y[tr[:, 1]])
    same = np.tile(y[3], (9, 1))
    half = np.full((3, 3), 1.0 / 3.0)
    assert np.allclose(O.combine_ref(same, np.array([[1, 2, 3]] * 3), half), np.tile(y[3], (3, 1)), rtol=1e-15)


def test_token_rows_invert_the_routing():
    ids, offs, row_token = W.moe_routing(37, E=20, topk=4, seed=5)
    tr = W.moe_token_rows(ids)
    assert tr.shape == (37, 4)
    assert np.array_equal(np.sort(tr.reshape(-1)), np.arange(37 * 4))
    for t in range(37):
        for k in range(4):
            r = tr[t, k]
            assert row_token[r] == t
            assert offs[ids[t, k]] <= r < offs[ids[t, k] + 1]
    w = W.moe_combine_weights(37, 4)
    assert w.dtype == np.float32 and np.all(w > 0) and np.allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    q, s = W.mx_bytes(5, 256, seed=1)
    assert q.shape == (5, 128) and s.shape == (5, 8) and s.min() >= 118 and s.max() < 130
