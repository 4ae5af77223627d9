"""GPU parity of the quantizers: the standalone activation quantizer and the weight
prepare must match the CPU oracle bit for bit (payload and scales)."""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import mx_oracle as O

from gpu_util import (dense_activation_cached, dense_weight_cached, dev_bf16, host_u8, lib_or_fail,
                      torch_or_skip)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")


def _quant_gpu(bits):
    mx = lib_or_fail()
    q, s = mx.mx_quant_act(dev_bf16(bits))
    return host_u8(q), host_u8(s)


@pytest.mark.parametrize("name,M", [("smoke_16x256x256", 16), ("n7168_k768", 2048), ("n7168_k4224", 2048),
                                    ("n7168_k4224", 3), ("n7168_k4224", 17), ("n7168_k4224", 100),
                                    ("n1536_k7168", 2048), ("n8448_k7168", 1)])
def test_quant_act_matches_oracle(name, M):
    torch_or_skip()
    a = dense_activation_cached(name, M)
    q, s = _quant_gpu(a)
    qo, so = O.quantize_mx(a)
    assert np.array_equal(s, so)
    assert np.array_equal(q, qo)


def test_quant_act_exhaustive_bf16_by_exponent():
    """Every finite bf16 value at every block exponent e in [-127, 125]: blocks of 31
    values with |x| < 2^(e+3) plus the anchor 2^(e+2), so the block exponent is e."""
    torch_or_skip()
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    xb = b[((b >> 7) & 0xFF) != 0xFF]
    x = O.bf16_to_f64(xb)
    rows = []
    for e in range(-127, 126):
        xs = xb[np.abs(x) < 2.0 ** (e + 3)]
        nblk = -(-xs.size // 31)
        flat = np.zeros(nblk * 31, dtype=np.uint16)
        flat[:xs.size] = xs
        blk = np.zeros((nblk, 32), dtype=np.uint16)
        blk[:, :31] = flat.reshape(nblk, 31)
        blk[:, 31] = W.f32_to_bf16_bits(np.array([2.0 ** (e + 2)], dtype=np.float32))[0]
        rows.append(blk)
    blocks = np.concatenate(rows)
    # pad the block count to a multiple of 8 and view as rows of K = 256
    pad = (-blocks.shape[0]) % 8
    blocks = np.concatenate([blocks, np.zeros((pad, 32), dtype=np.uint16)]).reshape(-1, 256)
    q, s = _quant_gpu(blocks)
    qo, so = O.quantize_mx(blocks)
    assert np.array_equal(s, so)
    assert np.array_equal(q, qo)


def test_quant_act_hand_worked_blocks():
    torch_or_skip()
    with open(GOLDEN) as f:
        blocks = json.load(f)["blocks"]
    bits = np.zeros((len(blocks), 32), dtype=np.uint16)
    for i, blk in enumerate(blocks):
        if "bits" in blk:
            head = [int(v, 16) for v in blk["bits"]]
        else:
            head = [0x8000 if v == "-0" else int(W.f32_to_bf16_bits(np.array([v], dtype=np.float32))[0])
                    for v in blk["values"]]
        bits[i, :len(head)] = head
    q, s = _quant_gpu(bits)
    codes = O.unpack_codes(q)
    for i, blk in enumerate(blocks):
        assert int(s[i, 0]) == blk["scale"], blk["name"]
        assert [int(c) for c in codes[i, :len(blk["codes_head"])]] == blk["codes_head"], blk["name"]
        if "payload_hex" in blk:
            assert q[i].tobytes().hex() == blk["payload_hex"], blk["name"]


@pytest.mark.parametrize("name", ["smoke_16x256x256", "n7168_k768", "n7168_k4224", "n1536_k7168",
                                  "n8448_k7168"])
def test_prepare_roundtrip_matches_oracle(name):
    """prepare -> unprepare gives the oracle's canonical quantization of W, bit for bit."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    N, K, _, _ = W.DENSE_CONFIGS[name]
    w, qo, so = dense_weight_cached(name)
    wp = mx.mx_prepare_weight(dev_bf16(w))
    assert wp.numel() == mx.mx_prepared_weight_bytes(N, K)
    q, s = mx.mx_unprepare_weight(wp, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(s), so)
    assert np.array_equal(host_u8(q), qo)


def test_prepare_moe_expert_shape():
    torch = torch_or_skip()
    mx = lib_or_fail()
    N, K = W.MOE_N, W.MOE_K
    w = W.moe_expert_weight(5)
    wp = mx.mx_prepare_weight(dev_bf16(w))
    assert wp.numel() == 2_924_544
    q, s = mx.mx_unprepare_weight(wp, N, K)
    torch.cuda.synchronize()
    qo, so = O.quantize_mx(w)
    assert np.array_equal(host_u8(s), so) and np.array_equal(host_u8(q), qo)


def test_prepared_layout_scale_words():
    """Scale word (quad q, step t, lane l) byte j is the scale of column 16(4q+j) + l%16 and
    K block 4t + l/16 (checked against the oracle's canonical scales, K = 4224 = 33 steps)."""
    torch_or_skip()
    mx = lib_or_fail()
    N, K = 256, 4224
    w = W.dense_weight(N, K, seed=77)
    wp = host_u8(mx.mx_prepare_weight(dev_bf16(w)))
    assert wp.size == N * K * 17 // 32
    _, so = O.quantize_mx(w)
    T = K // 128
    words = wp[N * K // 2:].view(np.uint32).reshape(N // 64, T, 64)
    for q in range(N // 64):
        for t in (0, 7, T - 1):
            for l in (0, 17, 63):
                for j in range(4):
                    n, kb = 16 * (4 * q + j) + l % 16, 4 * t + l // 16
                    assert (int(words[q, t, l]) >> (8 * j)) & 0xFF == so[n, kb]
