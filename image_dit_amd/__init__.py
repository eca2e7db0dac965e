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
"Quick start" -- read the device pointer out of existing tensors and call the
kernel on it, with no staging copies and no second GPU context.
"""
import ctypes
import os

__all__ = ["DitAttnError", "load", "abi_version", "sage_padded_len", "attn_fwd_bf16",
           "sage_prepare", "sage_attn_fwd", "sage_attention", "HEAD_DIM", "LIB_PATH"]

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
    for name in ("attn_fwd_bf16", "sage_prepare", "sage_attn_fwd"):
        getattr(lib, name).restype = ci
    _lib = lib
    return lib


def _status(lib, func, st):
    if st != 0:
        raise DitAttnError(func, st, lib.ditattn_status_string(st).decode())


def abi_version():
    return load().ditattn_abi_version()


def sage_padded_len(S):
    n = load().ditattn_sage_padded_len(int(S))
    if n < 0:
        raise ValueError("invalid sequence length %r" % (S,))
    return n


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(tensors, stream):
    """Tell the caching allocator that `stream` uses tensors this module
    allocated on the current stream, so it does not hand their memory out
    again before the work enqueued on `stream` has finished."""
    import torch
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        t.record_stream(stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check_bshd(name, t, dtype):
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError("%s must be a GPU tensor" % name)
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


def _prepared_specs(B, S, H, D):
    """(name, shape, dtype) of the six tensors sage_prepare writes."""
    import torch
    Sp = sage_padded_len(S)
    return (("q_i8", (B, H, Sp, D), torch.int8), ("q_scale", (B, H, Sp // 32), torch.float32),
            ("k_i8", (B, H, Sp, D), torch.int8), ("k_scale", (B, H, Sp // 32), torch.float32),
            ("v_fp8", (B, H, D, Sp), torch.uint8), ("v_scale", (B, H, D), torch.float32))


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
        _check_bshd(name, t, torch.bfloat16)
        if tuple(t.shape) != (B, S, H, D):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), (B, S, H, D)))
    if out is None:
        out = torch.empty_like(q)
        _on_stream([out], stream)
    else:
        _check_out("out", out, (B, S, H, D), torch.bfloat16, q.device)
    st = lib.attn_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, H, D, float(scale),
                           _stream_handle(stream))
    _status(lib, "attn_fwd_bf16", st)
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
        _check_bshd(name, t, torch.bfloat16)
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
    st = lib.sage_prepare(_ptr(q), _ptr(k), _ptr(v), *[_ptr(t) for t in out], B, S, H, D,
                          float(scale), _stream_handle(stream))
    _status(lib, "sage_prepare", st)
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
    st = lib.sage_attn_fwd(*[_ptr(t) for t in prepared], _ptr(out), B, int(S), int(H), D,
                           float(scale), _stream_handle(stream))
    _status(lib, "sage_attn_fwd", st)
    return out


def sage_attention(q, k, v, scale, stream=None):
    """sage_prepare followed by sage_attn_fwd."""
    B, S, H, D = _dims(q)
    prepared = sage_prepare(q, k, v, scale, stream=stream)
    return sage_attn_fwd(prepared, S, H, scale, stream=stream)
