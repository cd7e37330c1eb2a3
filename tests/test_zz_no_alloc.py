"""The allocation-free forward (moe_a16w4_forward_noalloc, for callers that
cannot allocate device memory) against the forward with a caller-allocated
workspace (moe_a16w4_forward): same inputs, same kernels, so the outputs
must agree bit for bit -- on two calls in a row, the second with a smaller
batch (the scratch still holds the first call's data), at the production
expert-parallel shape. Neither call may allocate device memory.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_grouped_gemm_amd as m
    return m


def _inputs(moe, wl, T, dev):
    s = wl.spec
    x = torch.from_numpy(wl.x[:T].view(np.int16).copy()).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(wl.logits[:T].copy()).to(dev)
    bm = moe.moe_default_block_m(T, s.topk, s.E)
    ids, w, srt, be, _, npp = moe.moe_route_align(logits, s.topk, s.E, bm)
    return x, ids, w, srt, be, npp, bm


def test_noalloc_matches_forward_two_calls(moe):
    dev = torch.device("cuda")
    wl = synth.make(synth.specs()["decode_t32"])
    s = wl.spec
    w13, w13s, w2, w2s = (torch.from_numpy(a).to(dev) for a in (wl.w13, wl.w13_scale, wl.w2, wl.w2_scale))
    cases = []
    # 32-row MFMA tiles, then 16-row blocks on the matrix-core kernels (with
    # the activations shared by the workgroup, then per wave): each call
    # smaller than the one before.
    for T in (32, 16, 3):
        x, ids, w, srt, be, npp, bm = _inputs(moe, wl, T, dev)
        ref = moe.moe_a16w4_forward(x, w13, w13s, w2, w2s, ids, w, srt, be, npp, bm)
        out = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
        cases.append((T, x, ids, w, srt, be, npp, bm, ref, out))
    torch.cuda.synchronize()
    # Warm-up outside the measured region: the first call on this device
    # looks up the scratch address, and the first launch of any kernel
    # (torch's fill included) loads its code object, which takes device
    # memory once per process.
    for T, x, ids, w, srt, be, npp, bm, ref, out in cases:
        out.fill_(float("nan"))
        moe.moe_a16w4_forward_noalloc(x, w13, w13s, w2, w2s, ids, w, srt, be, npp, bm, out)
    torch.cuda.synchronize()
    for T, x, ids, w, srt, be, npp, bm, ref, out in cases:
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        # device memory around the call alone (torch's own comparisons below
        # may grow its caching allocator's pool)
        alloc0 = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        free0 = torch.cuda.mem_get_info()[0]
        moe.moe_a16w4_forward_noalloc(x, w13, w13s, w2, w2s, ids, w, srt, be, npp, bm, out)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        assert free1 == free0, f"T={T}: free device memory changed by {free0 - free1} bytes"
        assert torch.cuda.max_memory_allocated() == alloc0
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"T={T}"


def test_noalloc_rejects_batches_beyond_scratch(moe):
    """A batch whose workspace exceeds the scratch fails before any launch."""
    s = synth.specs()["prefill_t1024"]
    T, bm = s.T, 32
    need = moe.moe_a16w4_workspace_size(T, s.H, s.I, s.E, s.topk, bm)
    assert need > moe.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda")
    x = torch.zeros((T, s.H), dtype=torch.bfloat16, device=dev)
    w13 = torch.zeros((s.E, 2 * s.I, s.H // 2), dtype=torch.uint8, device=dev)
    w13s = torch.zeros((s.E, 2 * s.I, s.H // 32), dtype=torch.uint8, device=dev)
    w2 = torch.zeros((s.E, s.H, s.I // 2), dtype=torch.uint8, device=dev)
    w2s = torch.zeros((s.E, s.H, s.I // 32), dtype=torch.uint8, device=dev)
    ids = torch.zeros((T, s.topk), dtype=torch.int32, device=dev)
    w = torch.zeros((T, s.topk), dtype=torch.float32, device=dev)
    cap = moe.moe_align_sort_capacity(T, s.topk, s.E, bm)
    srt = torch.full((cap,), T * s.topk, dtype=torch.int32, device=dev)
    be = torch.full((cap // bm,), -1, dtype=torch.int32, device=dev)
    npp = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
    out.fill_(1.0)
    torch.cuda.synchronize()
    with pytest.raises(moe.MoeError, match="scratch"):
        moe.moe_a16w4_forward_noalloc(x, w13, w13s, w2, w2s, ids, w, srt, be, npp, bm, out)
    torch.cuda.synchronize()
    assert torch.all(out == 1.0)  # nothing ran
