"""Pins for the oracle's expert biases and GEMM1 clamp.

[P2] create_weights (vLLM mxfp4 API page): under has_bias the layer holds
w13_bias [E, 2I] and w2_bias [E, H] in bf16; get_fused_moe_quant_config
passes them to the kernel with the layer's swiglu_limit as the GEMM1 clamp
limit. Reading (the pages give no formula): gate/up = W13 x + w13_bias,
each clamped to [-limit, limit] when a limit is set, h = bf16(silu(gate) *
up), y = W2 h + w2_bias, out = sum_j weight_j * y_j.

Pins: numpy float64 matmuls over weights decoded by tests/decode_ref.py
(a dense single-expert MLP and a brute-force loop over experts), np.clip for
the clamp, and a closed form: with all-zero weights every y is exactly its
expert's w2 bias, so the output is the router-weighted sum of bias rows.
"""
import numpy as np
import torch
from scipy.special import expit

import synth
from tests.decode_ref import bf16_bits_to_f64, dequant_mxfp4


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _mlp(x, w13d, w2d, I, b13=None, b2=None, limit=0.0):
    g = w13d[:I] @ x
    u = w13d[I:] @ x
    if b13 is not None:
        g = g + b13[:I]
        u = u + b13[I:]
    if limit > 0:
        g = np.clip(g, -limit, limit)
        u = np.clip(u, -limit, limit)
    h = _bf16(g * expit(g) * u)
    y = w2d @ h
    return y if b2 is None else y + b2


def test_single_expert_bias_clamp_is_dense_mlp(orc):
    wl = synth.small(T=3, H=64, I=32, E=1, topk=1, seed=31)
    b13, b2 = synth.biases(1, 64, 32, seed=32)
    ids = np.zeros((3, 1), dtype=np.int32)
    w = np.ones((3, 1), dtype=np.float32)
    x = bf16_bits_to_f64(wl.x)
    w13d = dequant_mxfp4(wl.w13[0], wl.w13_scale[0])
    w2d = dequant_mxfp4(wl.w2[0], wl.w2_scale[0])
    b13f, b2f = bf16_bits_to_f64(b13[0]), bf16_bits_to_f64(b2[0])
    g_rms = float(np.sqrt(np.mean((w13d[:32] @ x.T) ** 2)))
    for limit in (0.0, 0.5 * g_rms, 1e30):
        out = orc.moe_forward(wl.x, wl.w13, wl.w13_scale, wl.w2, wl.w2_scale, orc.FMT_MXFP4, ids, w,
                              I=32, w13_bias=b13, w2_bias=b2, swiglu_limit=limit)
        want = np.stack([_mlp(x[t], w13d, w2d, 32, b13f, b2f, limit) for t in range(3)])
        np.testing.assert_allclose(out, want, rtol=1e-10, atol=1e-10 * np.abs(want).max())
    # the clamp at half the gate RMS changes the result; a huge limit does not
    plain = orc.moe_forward(wl.x, wl.w13, wl.w13_scale, wl.w2, wl.w2_scale, 0, ids, w, I=32,
                            w13_bias=b13, w2_bias=b2)
    huge = orc.moe_forward(wl.x, wl.w13, wl.w13_scale, wl.w2, wl.w2_scale, 0, ids, w, I=32,
                           w13_bias=b13, w2_bias=b2, swiglu_limit=1e30)
    half = orc.moe_forward(wl.x, wl.w13, wl.w13_scale, wl.w2, wl.w2_scale, 0, ids, w, I=32,
                           w13_bias=b13, w2_bias=b2, swiglu_limit=0.5 * g_rms)
    assert np.array_equal(plain, huge)
    assert np.abs(half - plain).max() > 1e-3 * np.abs(plain).max()


def test_brute_force_experts_with_bias(orc):
    """Several experts: each pair takes its own expert's bias rows."""
    wl = synth.small(T=5, H=128, I=64, E=6, topk=3, seed=33)
    b13, b2 = synth.biases(6, 128, 64, seed=34)
    ids, w = orc.route_topk(wl.logits, 3)
    out = orc.moe_forward(wl.x, wl.w13, wl.w13_scale, wl.w2, wl.w2_scale, 0, ids, w, I=64,
                          w13_bias=b13, w2_bias=b2, swiglu_limit=80.0)
    x = bf16_bits_to_f64(wl.x)
    d13 = dequant_mxfp4(wl.w13, wl.w13_scale)
    d2 = dequant_mxfp4(wl.w2, wl.w2_scale)
    b13f, b2f = bf16_bits_to_f64(b13), bf16_bits_to_f64(b2)
    want = np.zeros((5, 128))
    for t in range(5):
        for j in range(3):
            e = ids[t, j]
            want[t] += float(w[t, j]) * _mlp(x[t], d13[e], d2[e], 64, b13f[e], b2f[e], 80.0)
    np.testing.assert_allclose(out, want, rtol=1e-9, atol=1e-9 * np.abs(want).max())


def test_zero_weights_give_weighted_bias_rows(orc):
    """All-zero weight codes: gate/up are exactly the w13 biases and every y
    is exactly its expert's w2 bias row, so out[t] = sum_j w[t, j] *
    w2_bias[ids[t, j]] (closed form, float64 sums of the same terms)."""
    wl = synth.small(T=4, H=64, I=32, E=5, topk=2, seed=35)
    b13, b2 = synth.biases(5, 64, 32, seed=36)
    z13 = np.zeros_like(wl.w13)
    z2 = np.zeros_like(wl.w2)
    ids, w = orc.route_topk(wl.logits, 2)
    out = orc.moe_forward(wl.x, z13, wl.w13_scale, z2, wl.w2_scale, 0, ids, w, I=32,
                          w13_bias=b13, w2_bias=b2, swiglu_limit=3.0)
    b2f = bf16_bits_to_f64(b2)
    want = np.zeros((4, 64))
    for t in range(4):
        for j in range(2):
            want[t] += float(w[t, j]) * b2f[ids[t, j]]
    assert np.array_equal(out, want)
