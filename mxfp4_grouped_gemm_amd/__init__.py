"""A16W4 mixture-of-experts layer for AMD MI355X (gfx950).

Thin ctypes binding over libmoe_a16w4.so (include/moe_a16w4.h). Every step
of the layer runs in the library's HIP kernels; this module only checks
tensor dtypes/devices, passes device pointers and the current HIP stream,
and turns a non-OK status into MoeError. PyTorch provides device memory and
streams. There is no CPU fallback: importing this package fails if the
library has not been built.

Functions mirror the C ABI names:
  moe_route_topk, moe_align_sort_capacity, moe_default_block_m,
  moe_align_sort, moe_route_align, moe_a16w4_workspace_size, moe_a16w4_forward,
  moe_a16w4_forward_stages, moe_a16w4_forward_ex, moe_a16w4_forward_monolithic,
  moe_a16w4_forward_noalloc,
  mxfp4_to_int4g32_requant, moe_last_error
plus two compositions: moe_a16w4_layer (route -> sort -> forward, the
in-kernel routing path of apply_monolithic on the vLLM mxfp4 API page) and
requantize_mxfp4_experts (the chunked MXFP4 -> int4-g32 load-time
conversion, eight experts per call).
"""
import contextlib
import ctypes
import os
import warnings

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_a16w4.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 0, 1, 2, 3
MOE_W_MXFP4, MOE_W_INT4G32 = 0, 1
MOE_ACT_SWIGLU = 0
MOE_STAGE_GATE_UP, MOE_STAGE_DOWN, MOE_STAGE_COMBINE, MOE_STAGE_ALL = 1, 2, 4, 7

# Every symbol include/moe_a16w4.h declares.
EXPORTS = (
    "moe_last_error", "moe_route_topk", "moe_align_sort_capacity", "moe_default_block_m",
    "moe_align_sort", "moe_route_align", "moe_a16w4_workspace_size", "moe_a16w4_forward",
    "moe_a16w4_forward_stages", "moe_a16w4_forward_ex", "moe_a16w4_forward_monolithic",
    "moe_a16w4_forward_noalloc",
    "mxfp4_to_int4g32_requant",
)
# Scratch of the allocation-free forward (MOE_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()'). There is no CPU fallback.")
    L = ctypes.CDLL(LIB_PATH)
    p, i, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_route_topk.restype = i
    L.moe_route_topk.argtypes = [p, i, i, i, i, p, p, p]
    L.moe_align_sort_capacity.restype = i64
    L.moe_align_sort_capacity.argtypes = [i, i, i, i]
    L.moe_default_block_m.restype = i
    L.moe_default_block_m.argtypes = [i, i, i]
    L.moe_align_sort.restype = i
    L.moe_align_sort.argtypes = [p, i, i, i, i, p, p, p, p, p]
    L.moe_route_align.restype = i
    L.moe_route_align.argtypes = [p, i, i, i, i, i, p, p, p, p, p, p, p]
    L.moe_a16w4_workspace_size.restype = i64
    L.moe_a16w4_workspace_size.argtypes = [i, i, i, i, i, i]
    L.moe_a16w4_forward.restype = i
    L.moe_a16w4_forward.argtypes = [p, p, p, p, p, i, i, p, p, p, p, p, i, i, i, i, i, i, p, p, sz, p]
    L.moe_a16w4_forward_stages.restype = i
    L.moe_a16w4_forward_stages.argtypes = [p, p, p, p, p, i, i, p, p, p, p, p, i, i, i, i, i, i, p, p, sz,
                                           ctypes.c_uint, p]
    L.moe_a16w4_forward_ex.restype = i
    L.moe_a16w4_forward_ex.argtypes = [p, p, p, p, p, p, p, i, i, ctypes.c_float, p, p, p, p, p, i, i, i, i,
                                       i, i, p, p, sz, ctypes.c_uint, p]
    L.moe_a16w4_forward_monolithic.restype = i
    L.moe_a16w4_forward_monolithic.argtypes = [p, p, p, p, p, p, p, p, i, i, ctypes.c_float, i, i, i, i, i,
                                               i, i, p, p, p, p, p, p, p, p, sz, ctypes.c_uint, p]
    L.moe_a16w4_forward_noalloc.restype = i
    L.moe_a16w4_forward_noalloc.argtypes = [p, p, p, p, p, i, i, p, p, p, p, p, i, i, i, i, i, i, p, p]
    L.mxfp4_to_int4g32_requant.restype = i
    L.mxfp4_to_int4g32_requant.argtypes = [p, p, i, i, i, i, i, p, p, p]
    return L


lib = _load()


def moe_last_error() -> str:
    return lib.moe_last_error().decode()


def _check(status):
    if status != MOE_OK:
        raise MoeError(status, moe_last_error())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocation context for the tensors a call creates: with an explicit
    stream they are allocated on it, so the caching allocator does not hand
    their memory to other work while the call's kernels still use it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dev(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def moe_route_topk(logits, topk, renormalize=True, topk_ids=None, topk_weights=None, stream=None):
    """Softmax top-k routing of fp32 logits [T, E] -> (ids int32, weights fp32) [T, topk]."""
    _dev(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    with _on(stream):
        if topk_ids is None:
            topk_ids = torch.empty((T, topk), dtype=torch.int32, device=logits.device)
        if topk_weights is None:
            topk_weights = torch.empty((T, topk), dtype=torch.float32, device=logits.device)
    _dev(topk_ids, "topk_ids", torch.int32)
    _dev(topk_weights, "topk_weights", torch.float32)
    _check(lib.moe_route_topk(_ptr(logits), T, E, int(topk), int(bool(renormalize)),
                              _ptr(topk_ids), _ptr(topk_weights), _stream(stream)))
    return topk_ids, topk_weights


def moe_align_sort_capacity(T, topk, E, block_m) -> int:
    return int(lib.moe_align_sort_capacity(int(T), int(topk), int(E), int(block_m)))


def moe_default_block_m(T, topk, E) -> int:
    return int(lib.moe_default_block_m(int(T), int(topk), int(E)))


def moe_align_sort(topk_ids, E, block_m, out=None, stream=None):
    """Group pairs by expert -> (sorted_ids, block_expert, expert_offsets, num_post_pad)."""
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    T, topk = topk_ids.shape
    cap = moe_align_sort_capacity(T, topk, E, block_m)
    if cap < 0:
        raise MoeError(MOE_ERR_INVALID_ARG, f"invalid align/sort sizes T={T} topk={topk} E={E} block_m={block_m}")
    dev = topk_ids.device
    if out is None:
        with _on(stream):
            out = (torch.empty(max(cap, 1), dtype=torch.int32, device=dev),
                   torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev),
                   torch.empty(E + 1, dtype=torch.int32, device=dev),
                   torch.empty(1, dtype=torch.int32, device=dev))
    sorted_ids, block_expert, offsets, npp = out
    if sorted_ids.numel() < cap or block_expert.numel() < cap // block_m or offsets.numel() < E + 1:
        raise ValueError("align/sort output buffers too small")
    _check(lib.moe_align_sort(_ptr(topk_ids), T, topk, int(E), int(block_m), _ptr(sorted_ids),
                              _ptr(block_expert), _ptr(offsets), _ptr(npp), _stream(stream)))
    return sorted_ids, block_expert, offsets, npp


def moe_route_align(logits, topk, E, block_m, renormalize=True, ids=None, weights=None, out=None,
                    stream=None):
    """Routing + align/sort in one call -> (ids, weights, sorted_ids, block_expert,
    expert_offsets, num_post_pad); identical to moe_route_topk then moe_align_sort."""
    _dev(logits, "logits", torch.float32, 2)
    T, El = logits.shape
    if El != E:
        raise ValueError(f"logits have {El} experts, expected {E}")
    dev = logits.device
    with _on(stream):
        if ids is None:
            ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
        if weights is None:
            weights = torch.empty((T, topk), dtype=torch.float32, device=dev)
    _dev(ids, "ids", torch.int32)
    _dev(weights, "weights", torch.float32)
    cap = moe_align_sort_capacity(T, topk, E, block_m)
    if cap < 0:
        raise MoeError(MOE_ERR_INVALID_ARG, f"invalid sizes T={T} topk={topk} E={E} block_m={block_m}")
    if out is None:
        with _on(stream):
            out = (torch.empty(max(cap, 1), dtype=torch.int32, device=dev),
                   torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev),
                   torch.empty(E + 1, dtype=torch.int32, device=dev),
                   torch.empty(1, dtype=torch.int32, device=dev))
    sorted_ids, block_expert, offsets, npp = out
    if sorted_ids.numel() < cap or block_expert.numel() < cap // block_m or offsets.numel() < E + 1:
        raise ValueError("align/sort output buffers too small")
    _check(lib.moe_route_align(_ptr(logits), T, int(E), int(topk), int(bool(renormalize)),
                               int(block_m), _ptr(ids), _ptr(weights), _ptr(sorted_ids),
                               _ptr(block_expert), _ptr(offsets), _ptr(npp), _stream(stream)))
    return ids, weights, sorted_ids, block_expert, offsets, npp


def moe_a16w4_workspace_size(T, H, I, E, topk, block_m) -> int:
    return int(lib.moe_a16w4_workspace_size(int(T), int(H), int(I), int(E), int(topk), int(block_m)))


def _weights(w13, w13_scale, w2, w2_scale, fmt):
    sdt = torch.uint8 if fmt == MOE_W_MXFP4 else (torch.int16, torch.uint16, torch.bfloat16)
    _dev(w13, "w13", torch.uint8, 3)
    _dev(w2, "w2", torch.uint8, 3)
    _dev(w13_scale, "w13_scale", sdt, 3)
    _dev(w2_scale, "w2_scale", sdt, 3)
    E, I2, Hh = w13.shape
    H, I = Hh * 2, I2 // 2
    if (w2.shape != (E, H, I // 2) or w13_scale.shape != (E, 2 * I, H // 32)
            or w2_scale.shape != (E, H, I // 32)):
        raise ValueError(
            f"weight shapes disagree: w13 {tuple(w13.shape)}, w13_scale {tuple(w13_scale.shape)}, "
            f"w2 {tuple(w2.shape)}, w2_scale {tuple(w2_scale.shape)}")
    return E, H, I


def _bias(b, name, shape):
    if b is None:
        return None
    _dev(b, name, (torch.bfloat16, torch.int16, torch.uint16), 2)
    if tuple(b.shape) != shape:
        raise ValueError(f"{name} must have shape {shape}, got {tuple(b.shape)}")
    return b


def moe_a16w4_forward(x, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids,
                      block_expert, num_post_pad, block_m, fmt=MOE_W_MXFP4, act=MOE_ACT_SWIGLU,
                      out=None, workspace=None, stream=None, stages=MOE_STAGE_ALL,
                      w13_bias=None, w2_bias=None, swiglu_limit=0.0):
    """Fused MoE forward with precomputed routing. x bf16 [T, H] -> out bf16 [T, H].
    `stages` selects a subset of the launches (moe_a16w4_forward_stages).
    Optional expert biases w13_bias bf16 [E, 2I] and w2_bias bf16 [E, H], and
    swiglu_limit > 0 clamping gate and up to [-limit, limit]
    (moe_a16w4_forward_ex)."""
    _dev(x, "x", torch.bfloat16, 2)
    E, H, I = _weights(w13, w13_scale, w2, w2_scale, fmt)
    T = x.shape[0]
    if x.shape[1] != H:
        raise ValueError(f"x has {x.shape[1]} columns, weights expect H={H}")
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    _dev(topk_weights, "topk_weights", torch.float32, 2)
    topk = topk_ids.shape[1]
    need = moe_a16w4_workspace_size(T, H, I, E, topk, block_m)
    if need < 0:
        raise MoeError(MOE_ERR_INVALID_ARG, "invalid forward sizes")
    with _on(stream):
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _dev(out, "out", torch.bfloat16)
    _bias(w13_bias, "w13_bias", (E, 2 * I))
    _bias(w2_bias, "w2_bias", (E, H))
    if w13_bias is not None or w2_bias is not None or swiglu_limit:
        _check(lib.moe_a16w4_forward_ex(
            _ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w13_bias), _ptr(w2), _ptr(w2_scale), _ptr(w2_bias),
            int(fmt), int(act), float(swiglu_limit), _ptr(topk_ids), _ptr(topk_weights), _ptr(sorted_ids),
            _ptr(block_expert), _ptr(num_post_pad), T, H, I, E, topk, int(block_m), _ptr(out),
            _ptr(workspace), workspace.numel(), int(stages), _stream(stream)))
        return out
    args = (_ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), int(fmt), int(act),
            _ptr(topk_ids), _ptr(topk_weights), _ptr(sorted_ids), _ptr(block_expert),
            _ptr(num_post_pad), T, H, I, E, topk, int(block_m), _ptr(out), _ptr(workspace),
            workspace.numel())
    if stages == MOE_STAGE_ALL:
        _check(lib.moe_a16w4_forward(*args, _stream(stream)))
    else:
        _check(lib.moe_a16w4_forward_stages(*args, int(stages), _stream(stream)))
    return out


def moe_a16w4_forward_noalloc(x, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids,
                              block_expert, num_post_pad, block_m, out, fmt=MOE_W_MXFP4,
                              act=MOE_ACT_SWIGLU, stream=None):
    """moe_a16w4_forward into a caller-given `out`, with the library's own
    device scratch as the workspace: neither this function nor the library
    allocates device memory (for callers that cannot allocate). Calls that
    overlap in time on one GPU share that scratch and race."""
    _dev(x, "x", torch.bfloat16, 2)
    E, H, I = _weights(w13, w13_scale, w2, w2_scale, fmt)
    T = x.shape[0]
    if x.shape[1] != H:
        raise ValueError(f"x has {x.shape[1]} columns, weights expect H={H}")
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    _dev(topk_weights, "topk_weights", torch.float32, 2)
    _dev(out, "out", torch.bfloat16, 2)
    topk = topk_ids.shape[1]
    _check(lib.moe_a16w4_forward_noalloc(
        _ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), int(fmt), int(act),
        _ptr(topk_ids), _ptr(topk_weights), _ptr(sorted_ids), _ptr(block_expert), _ptr(num_post_pad),
        T, H, I, E, topk, int(block_m), _ptr(out), _stream(stream)))
    return out


class MonolithicBuffers:
    """Every device buffer of moe_a16w4_forward_monolithic for one shape:
    the routing and align/sort outputs, the workspace and the output."""

    def __init__(self, T, H, I, E, topk, block_m, device, stream=None):
        cap = moe_align_sort_capacity(T, topk, E, block_m)
        need = moe_a16w4_workspace_size(T, H, I, E, topk, block_m)
        if cap < 0 or need < 0:
            raise MoeError(MOE_ERR_INVALID_ARG, f"invalid sizes T={T} H={H} I={I} E={E} topk={topk} "
                           f"block_m={block_m}")
        self.block_m = block_m
        with _on(stream):
            self.ids = torch.empty((T, topk), dtype=torch.int32, device=device)
            self.weights = torch.empty((T, topk), dtype=torch.float32, device=device)
            self.sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=device)
            self.block_expert = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=device)
            self.expert_offsets = torch.empty(E + 1, dtype=torch.int32, device=device)
            self.num_post_pad = torch.empty(1, dtype=torch.int32, device=device)
            self.workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
            self.out = torch.empty((T, H), dtype=torch.bfloat16, device=device)


def moe_a16w4_forward_monolithic(x, router_logits, w13, w13_scale, w2, w2_scale, topk, fmt=MOE_W_MXFP4,
                                 act=MOE_ACT_SWIGLU, renormalize=True, block_m=None, bufs=None,
                                 w13_bias=None, w2_bias=None, swiglu_limit=0.0, stages=MOE_STAGE_ALL,
                                 stream=None):
    """The layer from router logits in one call (apply_monolithic): routing,
    align/sort and the forward. `bufs` (MonolithicBuffers) holds every
    device buffer; one is allocated on `stream` when not given. Returns
    bufs (bufs.out is the layer output; bufs.ids / bufs.weights the routing)."""
    _dev(x, "x", torch.bfloat16, 2)
    _dev(router_logits, "router_logits", torch.float32, 2)
    E, H, I = _weights(w13, w13_scale, w2, w2_scale, fmt)
    T = x.shape[0]
    if x.shape[1] != H or tuple(router_logits.shape) != (T, E):
        raise ValueError(f"x {tuple(x.shape)} / router_logits {tuple(router_logits.shape)} do not match "
                         f"H={H}, E={E}")
    bm = moe_default_block_m(T, topk, E) if block_m is None else int(block_m)
    if bufs is None:
        bufs = MonolithicBuffers(T, H, I, E, topk, bm, x.device, stream)
    elif bufs.block_m != bm:
        raise ValueError(f"buffers were sized for block_m={bufs.block_m}, not {bm}")
    _bias(w13_bias, "w13_bias", (E, 2 * I))
    _bias(w2_bias, "w2_bias", (E, H))
    b = bufs
    _check(lib.moe_a16w4_forward_monolithic(
        _ptr(x), _ptr(router_logits), _ptr(w13), _ptr(w13_scale), _ptr(w13_bias), _ptr(w2), _ptr(w2_scale),
        _ptr(w2_bias), int(fmt), int(act), float(swiglu_limit), int(bool(renormalize)), T, H, I, E, int(topk),
        bm, _ptr(b.ids), _ptr(b.weights), _ptr(b.sorted_ids), _ptr(b.block_expert), _ptr(b.expert_offsets),
        _ptr(b.num_post_pad), _ptr(b.out), _ptr(b.workspace), b.workspace.numel(), int(stages),
        _stream(stream)))
    return bufs


def moe_a16w4_layer(x, router_logits, w13, w13_scale, w2, w2_scale, topk, fmt=MOE_W_MXFP4,
                    renormalize=True, block_m=None, stream=None, w13_bias=None, w2_bias=None,
                    swiglu_limit=0.0):
    """route -> align/sort -> forward on one stream (no host synchronisation),
    through moe_a16w4_forward_monolithic. With an explicit `stream` every
    tensor the call creates is allocated on that stream (the routing and
    sort arrays, the workspace and the output), so their memory stays
    reserved until the stream's work is done; the caller orders any use of
    the output on another stream as usual."""
    return moe_a16w4_forward_monolithic(x, router_logits, w13, w13_scale, w2, w2_scale, topk, fmt=fmt,
                                        renormalize=renormalize, block_m=block_m, w13_bias=w13_bias,
                                        w2_bias=w2_bias, swiglu_limit=swiglu_limit, stream=stream).out


def mxfp4_to_int4g32_requant(w, scale_e8m0, expert_lo, expert_hi, w_int4, scale_bf16, stream=None):
    """Requantize experts [lo, hi) of MXFP4 w [E, N, K/2] into preallocated outputs."""
    _dev(w, "w", torch.uint8, 3)
    _dev(scale_e8m0, "scale_e8m0", torch.uint8, 3)
    _dev(w_int4, "w_int4", torch.uint8, 3)
    _dev(scale_bf16, "scale_bf16", (torch.int16, torch.uint16, torch.bfloat16), 3)
    E, N, Kh = w.shape
    K = Kh * 2
    if (scale_e8m0.shape != (E, N, K // 32) or w_int4.shape != w.shape
            or scale_bf16.shape != (E, N, K // 32)):
        raise ValueError("requant tensor shapes disagree")
    _check(lib.mxfp4_to_int4g32_requant(_ptr(w), _ptr(scale_e8m0), E, N, K, int(expert_lo),
                                        int(expert_hi), _ptr(w_int4), _ptr(scale_bf16),
                                        _stream(stream)))
    return w_int4, scale_bf16


_warned_lossy = False


def requantize_mxfp4_experts(w, scale_e8m0, chunk=8, stream=None):
    """Convert a whole MXFP4 expert tensor to int4-g32, `chunk` experts per call,
    into preallocated outputs (the conversion loop of the MXFP4-to-int4 pull
    request). Returns (codes uint8 [E, N, K/2], scales bf16 [E, N, K/32])."""
    global _warned_lossy
    if not _warned_lossy:
        warnings.warn("Requantizing MXFP4 experts to groupwise int4 (int4_per_group_32): "
                      "this conversion is lossy.", stacklevel=2)
        _warned_lossy = True
    E, N, Kh = w.shape
    with _on(stream):
        codes = torch.empty_like(w)
        scales = torch.empty((E, N, Kh * 2 // 32), dtype=torch.bfloat16, device=w.device)
    for lo in range(0, E, chunk):
        mxfp4_to_int4g32_requant(w, scale_e8m0, lo, min(lo + chunk, E), codes, scales, stream=stream)
    return codes, scales
