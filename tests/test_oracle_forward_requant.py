"""Pins for the oracle's MoE forward and MXFP4 -> int4-g32 requantization.

Forward: W4A16 semantics (get_fused_moe_quant_config on the vLLM mxfp4 API
page: bf16 activations, weights dequantized), fused gate_up rows [0, I) gate
and [I, 2I) up (create_weights), SwiGLU whose output enters the down GEMM as
bf16 (the BF16 x packed-int4 path of the MXFP4-to-int4 pull request), down
projection, router weights applied at the combine (apply()). Pins: numpy
float64 matmuls over weights decoded by tests/decode_ref.py, scipy's expit
for the sigmoid, torch's bf16 cast for the activation rounding.

Requant: convert() in Mxfp4MoEMethod._setup_kernel_k3_situ_gfx942 (decode,
scale, bf16 cast, per-1x32 int4 quant, pack); pinned by the closed-form code
table below (the e8m0 factor cancels, so codes depend on the nibbles only).
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

import synth
from tests.decode_ref import (E2M1_TABLE, bf16_bits_to_f64, dequant_int4g32, dequant_mxfp4,
                              unpack_nibbles)


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _mlp(x, w13d, w2d, I):
    g = w13d[:I] @ x
    u = w13d[I:] @ x
    h = _bf16(g * expit(g) * u)  # the down GEMM's activation operand is bf16 (A16W4)
    return w2d @ h


def test_forward_single_expert_is_dense_swiglu(orc):
    wl = synth.small(T=3, H=64, I=32, E=1, topk=1, seed=21)
    ids = np.zeros((3, 1), dtype=np.int32)
    w = np.ones((3, 1), dtype=np.float32)
    out = orc.moe_forward(wl.x, wl.w13, wl.w13_scale, wl.w2, wl.w2_scale, orc.FMT_MXFP4, ids, w, I=32)
    x = bf16_bits_to_f64(wl.x)
    w13d = dequant_mxfp4(wl.w13[0], wl.w13_scale[0])
    w2d = dequant_mxfp4(wl.w2[0], wl.w2_scale[0])
    want = np.stack([_mlp(x[t], w13d, w2d, 32) for t in range(3)])
    np.testing.assert_allclose(out, want, rtol=1e-10, atol=1e-10 * np.abs(want).max())


@pytest.mark.parametrize("fmt", [0, 1])
def test_forward_brute_force_tiny(orc, fmt):
    wl = synth.make(synth.specs()["tiny"])
    T, H, I, E, k = 4, 256, 128, 8, 2
    ids, w = orc.route_topk(wl.logits, k)
    if fmt == 0:
        w13, s13, w2, s2 = wl.w13, wl.w13_scale, wl.w2, wl.w2_scale
        d13 = dequant_mxfp4(w13, s13)
        d2 = dequant_mxfp4(w2, s2)
    else:
        rng = np.random.default_rng(9)
        w13, w2 = wl.w13, wl.w2
        s13 = torch.from_numpy(rng.standard_normal((E, 2 * I, H // 32)).astype(np.float32)).to(
            torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        s2 = torch.from_numpy(rng.standard_normal((E, H, I // 32)).astype(np.float32)).to(
            torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        d13 = dequant_int4g32(w13, s13)
        d2 = dequant_int4g32(w2, s2)
    out = orc.moe_forward(wl.x, w13, s13, w2, s2, fmt, ids, w, I=I)
    x = bf16_bits_to_f64(wl.x)
    want = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            want[t] += float(w[t, j]) * _mlp(x[t], d13[e], d2[e], I)
    np.testing.assert_allclose(out, want, rtol=1e-9, atol=1e-9 * np.abs(want).max())
    # token subset returns the same rows
    sub = orc.moe_forward(wl.x, w13, s13, w2, s2, fmt, ids, w, I=I, tokens=[3, 1])
    assert np.array_equal(sub, out[[3, 1]])


def test_forward_identical_experts_ignore_routing(orc):
    wl = synth.small(T=5, H=64, I=32, E=6, topk=3, seed=22)
    w13 = np.repeat(wl.w13[:1], 6, axis=0)
    s13 = np.repeat(wl.w13_scale[:1], 6, axis=0)
    w2 = np.repeat(wl.w2[:1], 6, axis=0)
    s2 = np.repeat(wl.w2_scale[:1], 6, axis=0)
    ids, w = orc.route_topk(wl.logits, 3)
    a = orc.moe_forward(wl.x, w13, s13, w2, s2, 0, ids, w, I=32)
    ids1 = np.zeros((5, 1), dtype=np.int32)
    b = orc.moe_forward(wl.x, w13[:1], s13[:1], w2[:1], s2[:1], 0, ids1, np.ones((5, 1), np.float32), I=32)
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-6 * np.abs(b).max())


# Closed-form requant table. For an MX group whose largest |e2m1| is M and
# whose e8m0 byte s is in the normal range, every bf16 value is
# m * 2^(s-127) exactly, so scale = bf16(M/7) * 2^(s-127) and the code of a
# magnitude m is rint(m / bf16(M/7)), independent of s.
# M -> (bf16(M/7), {|m|: code}) for the e2m1 magnitudes m <= M.
REQUANT_TABLE = {
    0.5: (0.0712890625, {0.0: 0, 0.5: 7}),
    1.0: (0.142578125, {0.0: 0, 0.5: 4, 1.0: 7}),
    1.5: (0.2138671875, {0.0: 0, 0.5: 2, 1.0: 5, 1.5: 7}),
    2.0: (0.28515625, {0.0: 0, 0.5: 2, 1.0: 4, 1.5: 5, 2.0: 7}),
    3.0: (0.427734375, {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 4, 2.0: 5, 3.0: 7}),
    4.0: (0.5703125, {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 7}),
    6.0: (0.85546875, {0.0: 0, 0.5: 1, 1.0: 1, 1.5: 2, 2.0: 2, 3.0: 4, 4.0: 5, 6.0: 7}),
}
E2M1_CODE = {float(abs(v)): c for c, v in enumerate(E2M1_TABLE[:8])}


def _pack(codes):
    codes = np.asarray(codes, dtype=np.uint8) & 0xF
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("M", sorted(REQUANT_TABLE))
@pytest.mark.parametrize("sbyte", [118, 123, 127, 128, 130])
def test_requant_closed_form_table(orc, M, sbyte):
    sM, codes_of = REQUANT_TABLE[M]
    mags = sorted(codes_of)
    rng = np.random.default_rng(int(M * 10) + sbyte)
    # one group of 32: contains M, then random magnitudes <= M with random signs
    m = np.array([M] + list(rng.choice(mags, size=31)), dtype=np.float64)
    neg = rng.integers(0, 2, size=32).astype(bool)
    neg[0] = bool(sbyte % 2)  # the max itself negative sometimes
    e2m1_codes = np.array([E2M1_CODE[v] | (8 if n else 0) for v, n in zip(m, neg)], dtype=np.uint8)
    w = _pack(e2m1_codes).reshape(1, 1, 16)
    s = np.array([[[sbyte]]], dtype=np.uint8)
    q, sc = orc.requant_int4g32(w, s)
    want_codes = np.array([(-codes_of[v] if n else codes_of[v]) for v, n in zip(m, neg)])
    got_codes = unpack_nibbles(q).astype(np.int64).reshape(32)
    got_codes = np.where(got_codes >= 8, got_codes - 16, got_codes)
    assert got_codes.tolist() == want_codes.tolist()
    want_scale = np.float32(sM * 2.0 ** (sbyte - 127))
    assert bf16_bits_to_f64(sc.reshape(1))[0] == want_scale


def test_requant_zero_group(orc):
    w = np.zeros((1, 2, 16), dtype=np.uint8)
    w[0, 1] = 0x88  # all negative zeros
    s = np.full((1, 2, 1), 120, dtype=np.uint8)
    q, sc = orc.requant_int4g32(w, s)
    assert np.all(q == 0) and np.all(sc == 0)


def test_requant_reconstruction_bound_and_chunks(orc):
    wl = synth.small(T=1, H=128, I=64, E=10, topk=2, seed=23, scale_lo=118, scale_hi=128)
    w, s = wl.w13, wl.w13_scale
    E, N, Kh = w.shape
    q_all, s_all = orc.requant_int4g32(w, s)
    v = dequant_mxfp4(w, s)  # exact bf16 values in this scale range
    r = dequant_int4g32(q_all, s_all)
    scale = np.repeat(bf16_bits_to_f64(s_all), 32, axis=-1)
    assert np.all(np.abs(r - v) <= scale / 2 + 1e-30)
    # the group max maps to +-7 steps
    amax = np.abs(v).reshape(E, N, -1, 32).max(-1)
    nz = amax > 0
    codes = unpack_nibbles(q_all).astype(np.int64)
    codes = np.where(codes >= 8, codes - 16, codes).reshape(E, N, -1, 32)
    assert np.all(np.abs(codes).max(-1)[nz] == 7)
    # chunked conversion (8 experts at a time) into preallocated outputs
    qc = np.full_like(q_all, 0xAA)
    sc = np.full_like(s_all, 0xBEEF)
    for lo in range(0, E, 8):
        orc.requant_int4g32(w, s, lo, min(lo + 8, E), out=(qc, sc))
    assert np.array_equal(qc, q_all) and np.array_equal(sc, s_all)
    # a partial range leaves other experts untouched
    qp = np.full_like(q_all, 0xAA)
    sp = np.full_like(s_all, 0xBEEF)
    orc.requant_int4g32(w, s, 2, 5, out=(qp, sp))
    assert np.array_equal(qp[2:5], q_all[2:5]) and np.all(qp[:2] == 0xAA) and np.all(qp[5:] == 0xAA)
    assert np.array_equal(sp[2:5], s_all[2:5]) and np.all(sp[5:] == 0xBEEF)
