"""image_dit_amd -- MI355X (gfx950) DiT flash self-attention, BF16 and Sage modes.

A thin ctypes binding over libditattn.so (C ABI in include/ditattn.h).  Every
step of the computation runs in the library's HIP kernels; this module only
checks tensor shapes/dtypes/devices, passes device pointers, sizes and the
current HIP stream, and turns non-zero status codes into DitAttnError.
PyTorch is used for device memory and streams only.

If the library is missing the calls raise: there is no CPU or eager
fallback.  Build it with `python -m image_dit_amd.build` (or
`__graft_entry__.build()`).

Pattern of the binding: "RDNAttention" README, sections "Overview" and
"Quick start" -- the kernels get the addresses of tensors that already live on
the GPU; nothing is copied and no GPU context of the binding's own is opened.
"""
import ctypes
import os

__all__ = ["DitAttnError", "load", "abi_version", "sage_padded_len", "sage_workspace_size",
           "attn_fwd_bf16", "attn_fwd_bf16_ex", "sage_prepare", "sage_prepare_ex",
           "qk_norm_rope_bf16", "sage_attn_fwd", "sage_attn_fwd_ex", "sage_attention",
           "sage_attention_ex", "sage_prepare_ex_noalloc", "attn_fwd_bf16_ws", "bf16_workspace_size",
           "sage_attn_fwd_ws", "sage_attn_workspace_size",
           "STATIC_SCRATCH_BYTES", "HEAD_DIM", "LIB_PATH"]

HEAD_DIM = 128
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libditattn.so")

_lib = None


class DitAttnError(RuntimeError):
    def __init__(self, func, status, msg):
        super().__init__("%s failed: status %d (%s)" % (func, status, msg))
        self.status = status


def load(path=None):
    """Load libditattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError("libditattn.so not found at %s: build it with "
                           "`python -m image_dit_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.ditattn_abi_version.restype = ci
    lib.ditattn_status_string.argtypes = [ci]
    lib.ditattn_status_string.restype = ctypes.c_char_p
    lib.ditattn_sage_padded_len.argtypes = [ci]
    lib.ditattn_sage_padded_len.restype = ci
    lib.attn_fwd_bf16.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, cf, vp]
    lib.sage_prepare.argtypes = [vp] * 9 + [ci, ci, ci, ci, cf, vp]
    lib.sage_attn_fwd.argtypes = [vp] * 7 + [ci, ci, ci, ci, cf, vp]
    lib.sage_prepare_ex.argtypes = ([vp] * 9 + [ci] * 6 + [cf, vp, vp, cf, vp, vp, ci, vp, vp,
                                                          ctypes.c_size_t, vp])
    lib.qk_norm_rope_bf16.argtypes = [vp, vp, ci, ci, ci, ci, vp, cf, vp, vp, ci, vp]
    lib.attn_fwd_bf16_ex.argtypes = [vp, vp, vp, vp] + [ci] * 6 + [cf, ci, ci, vp]
    lib.sage_prepare_ex_noalloc.argtypes = [vp] * 9 + [ci] * 6 + [cf, vp, vp, cf, vp, vp, ci, vp, vp]
    lib.attn_fwd_bf16_ws.argtypes = [vp, vp, vp, vp] + [ci] * 6 + [cf, ci, ci, vp, ctypes.c_size_t, vp]
    lib.ditattn_bf16_workspace_size.argtypes = [ci] * 7
    lib.ditattn_bf16_workspace_size.restype = ctypes.c_size_t
    lib.sage_attn_fwd_ex.argtypes = [vp] * 7 + [ci] * 6 + [cf, ci, ci, vp]
    lib.sage_attn_fwd_ws.argtypes = [vp] * 7 + [ci] * 6 + [cf, ci, ci, vp, ctypes.c_size_t, vp]
    lib.ditattn_sage_attn_workspace_size.argtypes = [ci] * 7
    lib.ditattn_sage_attn_workspace_size.restype = ctypes.c_size_t
    lib.ditattn_sage_workspace_size.argtypes = [ci, ci, ci]
    lib.ditattn_sage_workspace_size.restype = ctypes.c_size_t
    for name in ("attn_fwd_bf16", "sage_prepare", "sage_attn_fwd", "sage_prepare_ex",
                 "qk_norm_rope_bf16", "attn_fwd_bf16_ex", "sage_attn_fwd_ex",
                 "sage_prepare_ex_noalloc", "attn_fwd_bf16_ws", "sage_attn_fwd_ws"):
        getattr(lib, name).restype = ci
    _lib = lib
    return lib


def _status(lib, func, st):
    if st != 0:
        raise DitAttnError(func, st, lib.ditattn_status_string(st).decode())


def abi_version():
    return load().ditattn_abi_version()


STATIC_SCRATCH_BYTES = 16 << 20  # the library's static device scratch (sage_prepare_ex_noalloc)


def sage_padded_len(S):
    n = load().ditattn_sage_padded_len(int(S))
    if n < 0:
        raise ValueError("invalid sequence length %r" % (S,))
    return n


def sage_workspace_size(B, S_kv, H_kv):
    """Bytes of workspace sage_prepare_ex needs for K smoothing."""
    return int(load().ditattn_sage_workspace_size(int(B), int(S_kv), int(H_kv)))


def _stream_handle(stream, device=None):
    """The HIP stream to launch on: `stream`, or the current stream of `device`.  A stream
    of another device than the tensors' is refused (the kernels would run on the wrong GPU)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif device is not None and stream.device != device:
        raise ValueError("stream is on %s, the tensors on %s" % (stream.device, device))
    return ctypes.c_void_p(stream.cuda_stream)


def _on_device(device):
    """Make the tensors' GPU the current device for a library call: the library launches on
    the current device and sizes the split-tail grid and the static scratch by it."""
    import contextlib
    import torch
    if device is None or device.type != "cuda":
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _on_stream(tensors, stream):
    """Tell the caching allocator that `stream` uses tensors this module
    allocated on the current stream, so it does not hand their memory out
    again before the work enqueued on `stream` has finished."""
    import torch
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        t.record_stream(stream)


def _zeroed_workspace(nbytes, device, stream):
    """A zero-filled byte buffer for a split-tail call on `stream`: the fill runs on the
    current stream, so `stream` (when it is another one) waits for it before the kernel."""
    import torch
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        stream.wait_stream(torch.cuda.current_stream(device))
        buf.record_stream(stream)
    return buf


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check_bshd(name, t, dtype, device=None):
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError("%s must be a GPU tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_out(name, t, shape, dtype, device):
    """Full check of a caller-supplied output: the library cannot see buffer
    sizes, so a short buffer would be written past its end."""
    import torch
    if not isinstance(t, torch.Tensor) or t.device != device:
        raise ValueError("%s must be a tensor on %s" % (name, device))
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _prepared_specs(B, S, H, D, S_kv=None, H_kv=None):
    """(name, shape, dtype) of the six tensors sage_prepare writes (Q side with S, H;
    K and V sides with S_kv, H_kv, by default the same)."""
    import torch
    S_kv = S if S_kv is None else S_kv
    H_kv = H if H_kv is None else H_kv
    Sq, Sk = sage_padded_len(S), sage_padded_len(S_kv)
    return (("q_i8", (B, H, Sq, D), torch.int8), ("q_scale", (B, H, Sq // 32), torch.float32),
            ("k_i8", (B, H_kv, Sk, D), torch.int8), ("k_scale", (B, H_kv, Sk // 32), torch.float32),
            ("v_fp8", (B, H_kv, D, Sk), torch.uint8), ("v_scale", (B, H_kv, D), torch.float32))


def _check_workspace(t, nbytes, device):
    """A caller-supplied workspace: a contiguous tensor on the tensors' GPU, >= nbytes."""
    import torch
    if (not isinstance(t, torch.Tensor) or t.device != device or not t.is_contiguous()
            or t.numel() * t.element_size() < nbytes):
        raise ValueError("workspace must be a contiguous tensor on %s of >= %d bytes" % (device, nbytes))
    return t.numel() * t.element_size()


def _dims(q):
    if q.dim() != 4:
        raise ValueError("expected [B, S, H, D], got shape %s" % (tuple(q.shape),))
    return tuple(int(x) for x in q.shape)


def attn_fwd_bf16(q, k, v, scale, out=None, stream=None):
    """BF16 flash attention: softmax(q k^T * scale) v, tensors [B, S, H, 128]."""
    import torch
    lib = load()
    B, S, H, D = _dims(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bshd(name, t, torch.bfloat16, device=q.device)
        if tuple(t.shape) != (B, S, H, D):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), (B, S, H, D)))
    if out is None:
        out = torch.empty_like(q)
        _on_stream([out], stream)
    else:
        _check_out("out", out, (B, S, H, D), torch.bfloat16, q.device)
    with _on_device(q.device):
        st = lib.attn_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, H, D, float(scale),
                               _stream_handle(stream, q.device))
    _status(lib, "attn_fwd_bf16", st)
    return out


def attn_fwd_bf16_ex(q, k, v, scale, window=(-1, -1), out=None, stream=None):
    """BF16 attention with q [B, S_q, H, 128], k and v [B, S_kv, H_kv, 128] (H a
    multiple of H_kv) and a key window (window_left, window_right): query i sees
    key j when i + off - wl <= j <= i + off + wr, off = S_kv - S_q, -1 meaning no
    bound on that side ((-1, 0) is causal).  Rows that see no key are zeros."""
    import torch
    lib = load()
    B, S_q, H, D = _dims(q)
    _, S_kv, H_kv, _ = _dims(k)
    _check_bshd("q", q, torch.bfloat16)
    for name, t in (("k", k), ("v", v)):
        _check_bshd(name, t, torch.bfloat16, device=q.device)
        if tuple(t.shape) != (B, S_kv, H_kv, D):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), (B, S_kv, H_kv, D)))
    if out is None:
        out = torch.empty_like(q)
        _on_stream([out], stream)
    else:
        _check_out("out", out, (B, S_q, H, D), torch.bfloat16, q.device)
    with _on_device(q.device):
        st = lib.attn_fwd_bf16_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S_q, S_kv, H, H_kv, D,
                                  float(scale), int(window[0]), int(window[1]),
                                  _stream_handle(stream, q.device))
    _status(lib, "attn_fwd_bf16_ex", st)
    return out


def bf16_workspace_size(B, S_q, S_kv, H, H_kv, window=(-1, -1)):
    """Bytes of workspace attn_fwd_bf16_ws needs on the current device (0: no split)."""
    return int(load().ditattn_bf16_workspace_size(int(B), int(S_q), int(S_kv), int(H), int(H_kv),
                                                   int(window[0]), int(window[1])))


def attn_fwd_bf16_ws(q, k, v, scale, window=(-1, -1), out=None, workspace=None, stream=None):
    """attn_fwd_bf16_ex with a workspace that splits the last, partial round of query
    tiles over every compute unit (see bf16_workspace_size).  workspace: a contiguous
    device buffer of at least that many bytes, zero-filled before its first use
    (allocated zero-filled here when None).
    One workspace serves one call at a time."""
    import torch
    lib = load()
    B, S_q, H, D = _dims(q)
    _, S_kv, H_kv, _ = _dims(k)
    _check_bshd("q", q, torch.bfloat16)
    for name, t in (("k", k), ("v", v)):
        _check_bshd(name, t, torch.bfloat16, device=q.device)
        if tuple(t.shape) != (B, S_kv, H_kv, D):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), (B, S_kv, H_kv, D)))
    if out is None:
        out = torch.empty_like(q)
        _on_stream([out], stream)
    else:
        _check_out("out", out, (B, S_q, H, D), torch.bfloat16, q.device)
    with _on_device(q.device):  # the split plan depends on the device's compute units
        need = bf16_workspace_size(B, S_q, S_kv, H, H_kv, window)
    ws_bytes = 0
    if need:
        if workspace is None:
            workspace = _zeroed_workspace(need, q.device, stream)
        ws_bytes = _check_workspace(workspace, need, q.device)
    with _on_device(q.device):
        st = lib.attn_fwd_bf16_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S_q, S_kv, H, H_kv, D,
                                  float(scale), int(window[0]), int(window[1]),
                                  _ptr(workspace) if need else None, ws_bytes,
                                  _stream_handle(stream, q.device))
    _status(lib, "attn_fwd_bf16_ws", st)
    return out


def sage_prepare(q, k, v, scale, out=None, stream=None):
    """Quantize Q, K, V for sage_attn_fwd.

    Returns (q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale) with shapes
    [B,H,S_pad,128] int8, [B,H,S_pad/32] f32, the same for K,
    [B,H,128,S_pad] uint8 (e4m3 bytes), [B,H,128] f32.
    """
    import torch
    lib = load()
    B, S, H, D = _dims(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bshd(name, t, torch.bfloat16, device=q.device)
        if tuple(t.shape) != (B, S, H, D):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), (B, S, H, D)))
    specs = _prepared_specs(B, S, H, D)
    if out is None:
        out = tuple(torch.empty(shape, dtype=dt, device=q.device) for _, shape, dt in specs)
        _on_stream(out, stream)
    else:
        if len(out) != 6:
            raise ValueError("out must be the 6 tensors of a sage_prepare result")
        for t, (name, shape, dt) in zip(out, specs):
            _check_out(name, t, shape, dt, q.device)
    with _on_device(q.device):
        st = lib.sage_prepare(_ptr(q), _ptr(k), _ptr(v), *[_ptr(t) for t in out], B, S, H, D,
                              float(scale), _stream_handle(stream, q.device))
    _status(lib, "sage_prepare", st)
    return out


def _opt_ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_small(name, t, shape, dtype, device):
    if t is not None:
        _check_out(name, t, shape, dtype, device)


def sage_prepare_ex(q, k, v, scale, q_norm_w=None, k_norm_w=None, norm_eps=1e-6, rope_cos=None,
                    rope_sin=None, rope_dim=0, smooth_k=False, out=None, k_mean=None,
                    workspace=None, stream=None):
    """sage_prepare with the optional Q/K transform (RMSNorm weights [128] BF16,
    RoPE tables [>= max(S_q, S_kv), rope_dim] BF16), K smoothing and
    cross-attention / grouped-query shapes: q [B, S_q, H, 128], k and v
    [B, S_kv, H_kv, 128].  Returns the six prepared tensors, plus the K channel
    mean [B, H_kv, 128] fp32 when smooth_k."""
    import torch
    lib = load()
    B, S_q, H, D = _dims(q)
    _, S_kv, H_kv, _ = _dims(k)
    _check_bshd("q", q, torch.bfloat16)
    for name, t in (("k", k), ("v", v)):
        _check_bshd(name, t, torch.bfloat16, device=q.device)
        if tuple(t.shape) != (B, S_kv, H_kv, D):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), (B, S_kv, H_kv, D)))
    dev = q.device
    _check_small("q_norm_w", q_norm_w, (D,), torch.bfloat16, dev)
    _check_small("k_norm_w", k_norm_w, (D,), torch.bfloat16, dev)
    if rope_dim:
        n_tab = max(S_q, S_kv)
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            if t is None or t.dim() != 2 or t.shape[0] < n_tab or t.shape[1] != rope_dim:
                raise ValueError("%s must be [>= %d, %d]" % (name, n_tab, rope_dim))
            _check_out(name, t, tuple(t.shape), torch.bfloat16, dev)
    specs = _prepared_specs(B, S_q, H, D, S_kv, H_kv)
    if out is None:
        out = tuple(torch.empty(shape, dtype=dt, device=dev) for _, shape, dt in specs)
        _on_stream(out, stream)
    else:
        if len(out) != 6:
            raise ValueError("out must be the 6 tensors of a sage_prepare result")
        for t, (name, shape, dt) in zip(out, specs):
            _check_out(name, t, shape, dt, dev)
    ws_bytes = 0
    if smooth_k:
        if k_mean is None:
            k_mean = torch.empty((B, H_kv, D), dtype=torch.float32, device=dev)
            _on_stream([k_mean], stream)
        _check_out("k_mean", k_mean, (B, H_kv, D), torch.float32, dev)
        ws_bytes = sage_workspace_size(B, S_kv, H_kv)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
            _on_stream([workspace], stream)
        ws_bytes = _check_workspace(workspace, ws_bytes, dev)
    else:
        k_mean = workspace = None
    with _on_device(dev):
        st = lib.sage_prepare_ex(_ptr(q), _ptr(k), _ptr(v), *[_ptr(t) for t in out], B, S_q, S_kv, H,
                                 H_kv, D, float(scale), _opt_ptr(q_norm_w), _opt_ptr(k_norm_w),
                                 float(norm_eps), _opt_ptr(rope_cos if rope_dim else None),
                                 _opt_ptr(rope_sin if rope_dim else None), int(rope_dim),
                                 _opt_ptr(k_mean), _opt_ptr(workspace), ws_bytes, _stream_handle(stream, dev))
    _status(lib, "sage_prepare_ex", st)
    return tuple(out) + ((k_mean,) if smooth_k else ())


def sage_prepare_ex_noalloc(q, k, v, scale, out, k_mean=None, q_norm_w=None, k_norm_w=None,
                            norm_eps=1e-6, rope_cos=None, rope_sin=None, rope_dim=0, stream=None):
    """sage_prepare_ex into caller-supplied outputs with no workspace: K smoothing
    (k_mean given, fp32 [B, H_kv, 128]) uses the library's static device scratch.
    The library allocates nothing; calls overlapping on one GPU race on that scratch."""
    import torch
    lib = load()
    B, S_q, H, D = _dims(q)
    _, S_kv, H_kv, _ = _dims(k)
    _check_bshd("q", q, torch.bfloat16)
    for name, t in (("k", k), ("v", v)):
        _check_bshd(name, t, torch.bfloat16, device=q.device)
        if tuple(t.shape) != (B, S_kv, H_kv, D):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), (B, S_kv, H_kv, D)))
    dev = q.device
    _check_small("q_norm_w", q_norm_w, (D,), torch.bfloat16, dev)
    _check_small("k_norm_w", k_norm_w, (D,), torch.bfloat16, dev)
    if rope_dim:
        n_tab = max(S_q, S_kv)
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            if t is None or t.dim() != 2 or t.shape[0] < n_tab or t.shape[1] != rope_dim:
                raise ValueError("%s must be [>= %d, %d]" % (name, n_tab, rope_dim))
            _check_out(name, t, tuple(t.shape), torch.bfloat16, dev)
    if out is None or len(out) != 6:
        raise ValueError("out must be the 6 preallocated tensors of a sage_prepare_ex result")
    for t, (name, shape, dt) in zip(out, _prepared_specs(B, S_q, H, D, S_kv, H_kv)):
        _check_out(name, t, shape, dt, dev)
    _check_small("k_mean", k_mean, (B, H_kv, D), torch.float32, dev)
    with _on_device(dev):
        st = lib.sage_prepare_ex_noalloc(_ptr(q), _ptr(k), _ptr(v), *[_ptr(t) for t in out], B, S_q,
                                         S_kv, H, H_kv, D, float(scale), _opt_ptr(q_norm_w),
                                         _opt_ptr(k_norm_w), float(norm_eps),
                                         _opt_ptr(rope_cos if rope_dim else None),
                                         _opt_ptr(rope_sin if rope_dim else None), int(rope_dim),
                                         _opt_ptr(k_mean), _stream_handle(stream, dev))
    _status(lib, "sage_prepare_ex_noalloc", st)
    return tuple(out) + ((k_mean,) if k_mean is not None else ())


def qk_norm_rope_bf16(x, norm_w=None, norm_eps=1e-6, rope_cos=None, rope_sin=None, rope_dim=0,
                      out=None, stream=None):
    """The Q/K row transform of sage_prepare_ex alone: BF16 [B, S, H, 128] in and out
    (out may be x itself)."""
    import torch
    lib = load()
    B, S, H, D = _dims(x)
    _check_bshd("x", x, torch.bfloat16)
    dev = x.device
    _check_small("norm_w", norm_w, (D,), torch.bfloat16, dev)
    if rope_dim:
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            if t is None or t.dim() != 2 or t.shape[0] < S or t.shape[1] != rope_dim:
                raise ValueError("%s must be [>= %d, %d]" % (name, S, rope_dim))
            _check_out(name, t, tuple(t.shape), torch.bfloat16, dev)
    if out is None:
        out = torch.empty_like(x)
        _on_stream([out], stream)
    else:
        _check_out("out", out, (B, S, H, D), torch.bfloat16, dev)
    with _on_device(dev):
        st = lib.qk_norm_rope_bf16(_ptr(x), _ptr(out), B, S, H, D, _opt_ptr(norm_w), float(norm_eps),
                                   _opt_ptr(rope_cos if rope_dim else None),
                                   _opt_ptr(rope_sin if rope_dim else None), int(rope_dim),
                                   _stream_handle(stream, dev))
    _status(lib, "qk_norm_rope_bf16", st)
    return out


def sage_attn_fwd(prepared, S, H, scale, out=None, stream=None):
    """The Sage forward on the tensors returned by sage_prepare; output [B, S, H, 128] BF16."""
    import torch
    lib = load()
    if len(prepared) != 6:
        raise ValueError("expected the 6 tensors returned by sage_prepare")
    q_i8 = prepared[0]
    if not isinstance(q_i8, torch.Tensor) or q_i8.dim() != 4 or q_i8.device.type != "cuda":
        raise ValueError("prepared tensors must be the GPU tensors returned by sage_prepare")
    B, D = int(q_i8.shape[0]), int(q_i8.shape[3])
    for t, (name, shape, dt) in zip(prepared, _prepared_specs(B, int(S), int(H), D)):
        _check_out(name, t, shape, dt, q_i8.device)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=q_i8.device)
        _on_stream([out], stream)
    else:
        _check_out("out", out, (B, S, H, D), torch.bfloat16, q_i8.device)
    with _on_device(q_i8.device):
        st = lib.sage_attn_fwd(*[_ptr(t) for t in prepared], _ptr(out), B, int(S), int(H), D,
                               float(scale), _stream_handle(stream, q_i8.device))
    _status(lib, "sage_attn_fwd", st)
    return out


def sage_attn_fwd_ex(prepared, S_q, S_kv, H, H_kv, scale, window=(-1, -1), out=None, stream=None):
    """The Sage forward on tensors from sage_prepare_ex, with the shapes and key
    window of attn_fwd_bf16_ex; output [B, S_q, H, 128] BF16."""
    import torch
    lib = load()
    if len(prepared) < 6:
        raise ValueError("expected the tensors returned by sage_prepare_ex")
    prepared = tuple(prepared[:6])
    q_i8 = prepared[0]
    if not isinstance(q_i8, torch.Tensor) or q_i8.dim() != 4 or q_i8.device.type != "cuda":
        raise ValueError("prepared tensors must be the GPU tensors returned by sage_prepare_ex")
    B, D = int(q_i8.shape[0]), int(q_i8.shape[3])
    for t, (name, shape, dt) in zip(prepared, _prepared_specs(B, int(S_q), int(H), D, int(S_kv), int(H_kv))):
        _check_out(name, t, shape, dt, q_i8.device)
    if out is None:
        out = torch.empty((B, S_q, H, D), dtype=torch.bfloat16, device=q_i8.device)
        _on_stream([out], stream)
    else:
        _check_out("out", out, (B, S_q, H, D), torch.bfloat16, q_i8.device)
    with _on_device(q_i8.device):
        st = lib.sage_attn_fwd_ex(*[_ptr(t) for t in prepared], _ptr(out), B, int(S_q), int(S_kv), int(H),
                                  int(H_kv), D, float(scale), int(window[0]), int(window[1]),
                                  _stream_handle(stream, q_i8.device))
    _status(lib, "sage_attn_fwd_ex", st)
    return out


def sage_attn_workspace_size(B, S_q, S_kv, H, H_kv, window=(-1, -1)):
    """Bytes of workspace sage_attn_fwd_ws needs on the current device (0: no split)."""
    return int(load().ditattn_sage_attn_workspace_size(int(B), int(S_q), int(S_kv), int(H), int(H_kv),
                                                        int(window[0]), int(window[1])))


def sage_attn_fwd_ws(prepared, S_q, S_kv, H, H_kv, scale, window=(-1, -1), out=None, workspace=None,
                     stream=None):
    """sage_attn_fwd_ex with a workspace that splits the last, partial round of query tiles
    over every compute unit (see sage_attn_workspace_size).  workspace: a contiguous buffer
    on the tensors' GPU of at least that many bytes, zero-filled before its first use
    (allocated zero-filled here when None).
    One workspace serves one call at a time."""
    import torch
    lib = load()
    if len(prepared) < 6:
        raise ValueError("expected the tensors returned by sage_prepare_ex")
    prepared = tuple(prepared[:6])
    q_i8 = prepared[0]
    if not isinstance(q_i8, torch.Tensor) or q_i8.dim() != 4 or q_i8.device.type != "cuda":
        raise ValueError("prepared tensors must be the GPU tensors returned by sage_prepare_ex")
    dev = q_i8.device
    B, D = int(q_i8.shape[0]), int(q_i8.shape[3])
    for t, (name, shape, dt) in zip(prepared, _prepared_specs(B, int(S_q), int(H), D, int(S_kv), int(H_kv))):
        _check_out(name, t, shape, dt, dev)
    if out is None:
        out = torch.empty((B, S_q, H, D), dtype=torch.bfloat16, device=dev)
        _on_stream([out], stream)
    else:
        _check_out("out", out, (B, S_q, H, D), torch.bfloat16, dev)
    with _on_device(dev):  # the split plan depends on the device's compute units
        need = sage_attn_workspace_size(B, S_q, S_kv, H, H_kv, window)
    ws_bytes = 0
    if need:
        if workspace is None:
            workspace = _zeroed_workspace(need, dev, stream)
        ws_bytes = _check_workspace(workspace, need, dev)
    with _on_device(dev):
        st = lib.sage_attn_fwd_ws(*[_ptr(t) for t in prepared], _ptr(out), B, int(S_q), int(S_kv), int(H),
                                  int(H_kv), D, float(scale), int(window[0]), int(window[1]),
                                  _ptr(workspace) if need else None, ws_bytes, _stream_handle(stream, dev))
    _status(lib, "sage_attn_fwd_ws", st)
    return out


def sage_attention_ex(q, k, v, scale, window=(-1, -1), smooth_k=False, stream=None, **xform):
    """sage_prepare_ex followed by sage_attn_fwd_ex (xform: the transform arguments of
    sage_prepare_ex)."""
    _, S_q, H, _ = _dims(q)
    _, S_kv, H_kv, _ = _dims(k)
    prepared = sage_prepare_ex(q, k, v, scale, smooth_k=smooth_k, stream=stream, **xform)
    return sage_attn_fwd_ex(prepared, S_q, S_kv, H, H_kv, scale, window, stream=stream)


def sage_attention(q, k, v, scale, stream=None):
    """sage_prepare followed by sage_attn_fwd."""
    B, S, H, D = _dims(q)
    prepared = sage_prepare(q, k, v, scale, stream=stream)
    return sage_attn_fwd(prepared, S, H, scale, stream=stream)
