"""CPU oracle for the DiT flash self-attention path.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports,
links or loads anything from this package, and this package never imports the
product library.

The arithmetic lives in oracle.c (plain C, fp64 attention, IEEE fp32
quantizer); this module only marshals numpy arrays through ctypes.  Inputs are
BF16 bit patterns as numpy uint16 arrays in [B, S, H, D] order.

Citations (page title, section):
  * exact attention: "Kernel acceleration: attention, compilation and fusion",
    section "Attention: from O(N^2) memory to blocks" (naive and blocked forms);
  * quantizer: "gfx1201_sage_prepare / gfx1201_sage_attention" (aiter PR 6390),
    section "Technical Details" (INT8 Q/K with one FP32 scale per 32-row block,
    Q carrying softmax_scale * log2(e); FP8 e4m3 V with one scale per channel,
    transposed to [B, H, 128, S_pad]);
  * Q/K row transform: the same page, first commit and "Technical Details"
    (optional RMSNorm and rotate-half RoPE, rope_dim 32/64/96/128, rounded like
    the eager PyTorch BF16 sequence);
  * attention of the quantized operands: the same page, commit text of
    gfx1201_sage_attention (INT8 Q K^T, FP8 P V, FP32 scales, online softmax in
    base 2), exact in fp64, without the rounding of P.
"""
import ctypes
import math
import os

import numpy as np

from . import build as _build

_LIB = None

LOG2E = 1.4426950408889634


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f64p = ctypes.POINTER(ctypes.c_double)
        i8p = ctypes.POINTER(ctypes.c_int8)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        f32p = ctypes.POINTER(ctypes.c_float)
        ci, cf = ctypes.c_int, ctypes.c_float
        lib.oracle_num_threads.restype = ci
        lib.oracle_softmax_row.argtypes = [u16p, u16p, ci, ci, ci, ci, cf, ci, ci, ci, f64p]
        lib.oracle_attn_rows.argtypes = [u16p, u16p, u16p, ci, ci, ci, ci, cf, i64p,
                                         ctypes.c_int64, f64p, ci]
        lib.oracle_attn_blocked.argtypes = [u16p, u16p, u16p, ci, ci, ci, ci, cf, ci, ci, f64p]
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [cf]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_sage_padded_len.argtypes = [ci]
        lib.oracle_sage_padded_len.restype = ci
        lib.oracle_quant_qk.argtypes = [u16p, ci, ci, ci, ci, cf, ci, i8p, f32p]
        lib.oracle_quant_v.argtypes = [u16p, ci, ci, ci, ci, ci, u8p, f32p]
        lib.oracle_quant_qk_mean.argtypes = [u16p, ci, ci, ci, ci, cf, ci, f32p, i8p, f32p]
        lib.oracle_channel_mean.argtypes = [u16p, ci, ci, ci, ci, f32p]
        lib.oracle_attn_rows_ex.argtypes = [u16p, u16p, u16p, ci, ci, ci, ci, ci, ci, cf, ci, ci,
                                            i64p, ctypes.c_int64, f64p, ci]
        lib.oracle_f32_to_bf16.argtypes = [cf]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_qk_norm_rope.argtypes = [u16p, ci, ci, ci, ci, u16p, cf, u16p, u16p, ci, u16p]
        lib.oracle_sage_attn_rows.argtypes = [i8p, f32p, i8p, f32p, u8p, f32p, ci, ci, ci, ci, ci,
                                              i64p, ctypes.c_int64, f64p, ci]
        lib.oracle_sage_attn_rows_ex.argtypes = [i8p, f32p, i8p, f32p, u8p, f32p, ci, ci, ci, ci, ci,
                                                 ci, ci, ci, ci, ci, i64p, ctypes.c_int64, f64p, ci]
        for name in ("oracle_softmax_row", "oracle_attn_rows", "oracle_attn_blocked",
                     "oracle_quant_qk", "oracle_quant_v", "oracle_qk_norm_rope",
                     "oracle_quant_qk_mean", "oracle_channel_mean", "oracle_attn_rows_ex",
                     "oracle_sage_attn_rows", "oracle_sage_attn_rows_ex"):
            getattr(lib, name).restype = ci
        _LIB = lib
    return _LIB


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _bits(x):
    """Accept a BF16 bit array (uint16/int16) or a torch bfloat16 tensor."""
    if hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch
        x = x.detach().cpu().contiguous().view(torch.int16).numpy()
    x = np.ascontiguousarray(x)
    if x.dtype == np.int16:
        x = x.view(np.uint16)
    if x.dtype != np.uint16:
        raise TypeError("expected BF16 bit patterns (uint16), got %s" % x.dtype)
    return x


def _check(status, what):
    if status != 0:
        raise RuntimeError("%s failed with oracle status %d" % (what, status))


def num_threads():
    return _lib().oracle_num_threads()


def q_multiplier(scale):
    """c = float32(double(scale) * log2(e)): the factor Q carries into INT8."""
    return float(np.float32(float(np.float32(scale)) * LOG2E))


def softmax_row(q, k, scale, b, h, i):
    """Probabilities p_j of query row (b, h, i) over all S keys (fp64)."""
    q, k = _bits(q), _bits(k)
    B, S, H, D = q.shape
    p = np.empty(S, dtype=np.float64)
    _check(_lib().oracle_softmax_row(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                     B, S, H, D, scale, b, h, i, _ptr(p, ctypes.c_double)),
           "oracle_softmax_row")
    return p


def attn_rows(q, k, v, scale, rows=None, nthreads=0):
    """Exact fp64 attention for the query rows `rows` (n x 3 array of b, h, i).

    rows=None means every row; the result then has shape [B, S, H, D], else
    [n, D].
    """
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, S, H, D = q.shape
    full = rows is None
    if full:
        b, i, h = np.meshgrid(np.arange(B), np.arange(S), np.arange(H), indexing="ij")
        rows = np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], D), dtype=np.float64)
    _check(_lib().oracle_attn_rows(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                   _ptr(v, ctypes.c_uint16), B, S, H, D, scale,
                                   _ptr(rows, ctypes.c_int64), rows.shape[0],
                                   _ptr(out, ctypes.c_double), nthreads),
           "oracle_attn_rows")
    if full:
        return out.reshape(B, S, H, D)
    return out


def attn_rows_ex(q, k, v, scale, window=(-1, -1), rows=None, nthreads=0):
    """Exact fp64 attention with q [B, S_q, H, D], k and v [B, S_kv, H_kv, D]
    (query head h reads key/value head h // (H // H_kv)) and a key window
    (wl, wr): query i sees key j when i + off - wl <= j <= i + off + wr,
    off = S_kv - S_q, a negative bound meaning none on that side.  A row that
    sees no key is 0.  rows: n x 3 (b, h, i) or None for every row ([B, S_q, H, D])."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, S_q, H, D = q.shape
    _, S_kv, H_kv, _ = k.shape
    full = rows is None
    if full:
        b, i, h = np.meshgrid(np.arange(B), np.arange(S_q), np.arange(H), indexing="ij")
        rows = np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], D), dtype=np.float64)
    _check(_lib().oracle_attn_rows_ex(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                      _ptr(v, ctypes.c_uint16), B, S_q, S_kv, H, H_kv, D, scale,
                                      int(window[0]), int(window[1]), _ptr(rows, ctypes.c_int64),
                                      rows.shape[0], _ptr(out, ctypes.c_double), nthreads),
           "oracle_attn_rows_ex")
    if full:
        return out.reshape(B, S_q, H, D)
    return out


def attn_blocked(q, k, v, scale, bq=64, bk=64):
    """Blocked online-softmax attention over every row, fp64, [B, S, H, D]."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, S, H, D = q.shape
    out = np.empty((B, S, H, D), dtype=np.float64)
    _check(_lib().oracle_attn_blocked(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                      _ptr(v, ctypes.c_uint16), B, S, H, D, scale, bq, bk,
                                      _ptr(out, ctypes.c_double)),
           "oracle_attn_blocked")
    return out


def e4m3_decode(code):
    return _lib().oracle_e4m3_decode(int(code) & 0xFF)


def e4m3_encode(x):
    return int(_lib().oracle_e4m3_encode(float(x)))


def sage_padded_len(S):
    return int(_lib().oracle_sage_padded_len(int(S)))


def quant_qk(x, mult, mean=None):
    """INT8 block quantization: codes [B, H, S_pad, D] int8, scales [B, H, S_pad/32] fp32.
    With mean (fp32 [B, H, D]) the values quantized are (fp32(x) - mean) * mult."""
    x = _bits(x)
    B, S, H, D = x.shape
    S_pad = sage_padded_len(S)
    codes = np.empty((B, H, S_pad, D), dtype=np.int8)
    scales = np.empty((B, H, S_pad // 32), dtype=np.float32)
    if mean is None:
        st = _lib().oracle_quant_qk(_ptr(x, ctypes.c_uint16), B, S, H, D, float(mult), S_pad,
                                    _ptr(codes, ctypes.c_int8), _ptr(scales, ctypes.c_float))
    else:
        mean = np.ascontiguousarray(mean, dtype=np.float32).reshape(B, H, D)
        st = _lib().oracle_quant_qk_mean(_ptr(x, ctypes.c_uint16), B, S, H, D, float(mult), S_pad,
                                         _ptr(mean, ctypes.c_float), _ptr(codes, ctypes.c_int8),
                                         _ptr(scales, ctypes.c_float))
    _check(st, "oracle_quant_qk")
    return codes, scales


def channel_mean(x):
    """fp32(fp64 sum over tokens / S) per (b, h, channel): fp32 [B, H, D]."""
    x = _bits(x)
    B, S, H, D = x.shape
    mean = np.empty((B, H, D), dtype=np.float32)
    _check(_lib().oracle_channel_mean(_ptr(x, ctypes.c_uint16), B, S, H, D, _ptr(mean, ctypes.c_float)),
           "oracle_channel_mean")
    return mean


def quant_v(v):
    """FP8 e4m3 per-channel quantization, transposed: codes [B, H, D, S_pad] uint8, scales [B, H, D]."""
    v = _bits(v)
    B, S, H, D = v.shape
    S_pad = sage_padded_len(S)
    codes = np.empty((B, H, D, S_pad), dtype=np.uint8)
    scales = np.empty((B, H, D), dtype=np.float32)
    _check(_lib().oracle_quant_v(_ptr(v, ctypes.c_uint16), B, S, H, D, S_pad,
                                 _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_float)),
           "oracle_quant_v")
    return codes, scales


def sage_prepare(q, k, v, scale):
    """The full prepare stage: (q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale)."""
    qc, qs = quant_qk(q, q_multiplier(scale))
    kc, ks = quant_qk(k, 1.0)
    vc, vs = quant_v(v)
    return qc, qs, kc, ks, vc, vs


def sage_attn_rows(prepared, S, rows, nthreads=0):
    """Attention of the quantized operands (q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale) as
    sage_prepare returns them, exact in fp64, for S real tokens and the query rows `rows`
    (n x 3 array of b, h, i): the scores are the INT8 dot products times both block scales, in
    base 2 (Q's scale carries softmax_scale * log2(e)); P V uses the decoded FP8 V times its
    channel scale.  Returns [n, D]."""
    qc, qs, kc, ks, vc, vs = (np.ascontiguousarray(a) for a in prepared)
    B, H, S_pad, D = qc.shape
    assert qc.dtype == np.int8 and kc.dtype == np.int8 and vc.dtype == np.uint8
    assert qs.dtype == np.float32 and ks.dtype == np.float32 and vs.dtype == np.float32
    assert kc.shape == qc.shape and vc.shape == (B, H, D, S_pad) and vs.shape == (B, H, D)
    assert qs.shape == ks.shape == (B, H, S_pad // 32) and 0 < S <= S_pad
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], D), dtype=np.float64)
    _check(_lib().oracle_sage_attn_rows(_ptr(qc, ctypes.c_int8), _ptr(qs, ctypes.c_float),
                                        _ptr(kc, ctypes.c_int8), _ptr(ks, ctypes.c_float),
                                        _ptr(vc, ctypes.c_uint8), _ptr(vs, ctypes.c_float),
                                        B, S, H, D, S_pad, _ptr(rows, ctypes.c_int64),
                                        rows.shape[0], _ptr(out, ctypes.c_double), nthreads),
           "oracle_sage_attn_rows")
    return out


def sage_attn_rows_ex(prepared, S_q, S_kv, window=(-1, -1), rows=None, nthreads=0):
    """sage_attn_rows for the prepared tensors of sage_prepare_ex: Q codes [B, H, S_q_pad, D],
    K/V of H_kv heads and S_kv real tokens (query head h reads head h // (H // H_kv)), and the
    key window of attn_rows_ex; a row that sees no key is 0.  Returns [n, D]."""
    qc, qs, kc, ks, vc, vs = (np.ascontiguousarray(a) for a in prepared[:6])
    B, H, S_q_pad, D = qc.shape
    _, H_kv, S_kv_pad, _ = kc.shape
    assert qc.dtype == np.int8 and kc.dtype == np.int8 and vc.dtype == np.uint8
    assert qs.dtype == np.float32 and ks.dtype == np.float32 and vs.dtype == np.float32
    assert vc.shape == (B, H_kv, D, S_kv_pad) and vs.shape == (B, H_kv, D)
    assert qs.shape == (B, H, S_q_pad // 32) and ks.shape == (B, H_kv, S_kv_pad // 32)
    assert 0 < S_q <= S_q_pad and 0 < S_kv <= S_kv_pad
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], D), dtype=np.float64)
    _check(_lib().oracle_sage_attn_rows_ex(_ptr(qc, ctypes.c_int8), _ptr(qs, ctypes.c_float),
                                           _ptr(kc, ctypes.c_int8), _ptr(ks, ctypes.c_float),
                                           _ptr(vc, ctypes.c_uint8), _ptr(vs, ctypes.c_float),
                                           B, S_q, S_kv, H, H_kv, D, S_q_pad, S_kv_pad,
                                           int(window[0]), int(window[1]),
                                           _ptr(rows, ctypes.c_int64), rows.shape[0],
                                           _ptr(out, ctypes.c_double), nthreads),
           "oracle_sage_attn_rows_ex")
    return out


def f32_to_bf16(x):
    """BF16 bits of fp32 x, round to nearest even (scalar)."""
    return int(_lib().oracle_f32_to_bf16(float(np.float32(x))))


def qk_norm_rope(x, norm_w=None, eps=1e-6, cos=None, sin=None, rope_dim=0):
    """RoPE(RMSNorm(x)) per (b, s, h) row with BF16 rounding after every step.

    x: BF16 [B, S, H, D]; norm_w: BF16 [D] or None; cos, sin: BF16
    [>= S, rope_dim] or None.  Returns the BF16 bits, uint16 [B, S, H, D].
    """
    x = _bits(x)
    B, S, H, D = x.shape
    null = ctypes.POINTER(ctypes.c_uint16)()
    w = _bits(norm_w) if norm_w is not None else None
    c = _bits(cos) if rope_dim else None
    s_ = _bits(sin) if rope_dim else None
    if rope_dim and (c.shape[-1] != rope_dim or s_.shape[-1] != rope_dim or c.shape[0] < S):
        raise ValueError("rope tables must be [>= S, rope_dim]")
    out = np.empty_like(x)
    _check(_lib().oracle_qk_norm_rope(
        _ptr(x, ctypes.c_uint16), B, S, H, D,
        _ptr(w, ctypes.c_uint16) if w is not None else null, float(eps),
        _ptr(c, ctypes.c_uint16) if rope_dim else null,
        _ptr(s_, ctypes.c_uint16) if rope_dim else null, int(rope_dim),
        _ptr(out, ctypes.c_uint16)), "oracle_qk_norm_rope")
    return out


def sage_prepare_ex(q, k, v, scale, q_norm_w=None, k_norm_w=None, eps=1e-6, cos=None,
                    sin=None, rope_dim=0, smooth_k=False):
    """The prepare stage with its options, by definition:
    Q' = qk_norm_rope(q), K' = qk_norm_rope(k) (each side's transform only when
    asked for), then the quantizer on Q', K' (minus K''s channel mean when
    smooth_k) and V.  Q and K/V may differ in tokens and heads.  Returns the
    six prepared arrays, plus the K channel mean when smooth_k."""
    xq = q_norm_w is not None or rope_dim
    xk = k_norm_w is not None or rope_dim
    qt = qk_norm_rope(q, q_norm_w, eps, cos, sin, rope_dim) if xq else _bits(q)
    kt = qk_norm_rope(k, k_norm_w, eps, cos, sin, rope_dim) if xk else _bits(k)
    mean = channel_mean(kt) if smooth_k else None
    qc, qs = quant_qk(qt, q_multiplier(scale))
    kc, ks = quant_qk(kt, 1.0, mean)
    vc, vs = quant_v(v)
    out = (qc, qs, kc, ks, vc, vs)
    return out + (mean,) if smooth_k else out
