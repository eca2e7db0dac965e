"""Algorithmic cost model of the attention path (FLOPs and HBM bytes).

"Kernel acceleration: attention, compilation and fusion", section
"Attention: from O(N^2) memory to blocks": the flash form reads Q, K, V and
writes O once (the scores stay on chip), while the naive form also writes the
N x N scores, reads them back and writes P.  Attention FLOPs are 4 * N^2 * d
per head (two GEMMs of 2 N^2 d), as in the block profile of section "The
memory-bound small operations: compilation and fusion"; the benchmark of
"gfx1201_sage_prepare / gfx1201_sage_attention", section "How to reproduce",
uses the same 4 * B * H * S^2 * 128 count.  Padding, masking and softmax work
are not counted.
"""


def sage_padded_len(S: int) -> int:
    """S rounded up to a multiple of 256 (the padded length of the prepared tensors)."""
    return (S + 255) // 256 * 256


def attn_flops(B: int, H: int, S: int, D: int = 128) -> float:
    return 4.0 * B * H * S * S * D


def score_matrix_bytes(B: int, H: int, S: int, dtype_bytes: int = 2) -> float:
    return float(B) * S * S * H * dtype_bytes


def attn_bytes_bf16(B: int, H: int, S: int, D: int = 128, dtype_bytes: int = 2) -> float:
    """Flash traffic: read Q, K, V and write O once."""
    return 4.0 * B * S * H * D * dtype_bytes


def naive_attn_bytes(B: int, H: int, S: int, D: int = 128, dtype_bytes: int = 2) -> float:
    """Naive traffic: write the scores, read them back, write P, plus Q, K, V and O."""
    return 2 * score_matrix_bytes(B, H, S, dtype_bytes) + attn_bytes_bf16(B, H, S, D, dtype_bytes)


def sage_prepare_bytes(B: int, H: int, S: int, D: int = 128) -> float:
    """Read Q, K, V (BF16) plus V a second time for its channel absmax; write the
    INT8 Q/K codes, the FP8 V codes (all padded to S_pad) and the FP32 scales."""
    Sp = sage_padded_len(S)
    read = 4.0 * B * S * H * D * 2
    write = 3.0 * B * H * Sp * D + 4.0 * (2 * B * H * (Sp // 32) + B * H * D)
    return read + write


def sage_attn_bytes(B: int, H: int, S: int, D: int = 128) -> float:
    """Read the 8-bit Q, K, V codes and their scales once, write BF16 O."""
    Sp = sage_padded_len(S)
    read = 3.0 * B * H * Sp * D + 4.0 * (2 * B * H * (Sp // 32) + B * H * D)
    return read + 2.0 * B * S * H * D


def visible_pairs(S_q: int, S_kv: int, window=(-1, -1)) -> int:
    """(query, key) pairs a key window leaves visible in one (b, h): query i sees key j when
    i + off - wl <= j <= i + off + wr with off = S_kv - S_q (a negative bound: none)."""
    wl, wr = window
    if wl < 0 and wr < 0:
        return S_q * S_kv
    import numpy as np
    i = np.arange(S_q, dtype=np.int64) + (S_kv - S_q)
    lo = np.zeros_like(i) if wl < 0 else np.maximum(i - wl, 0)
    hi = np.full_like(i, S_kv - 1) if wr < 0 else np.minimum(i + wr, S_kv - 1)
    return int(np.maximum(hi - lo + 1, 0).sum())


def attn_flops_ex(B: int, H: int, S_q: int, S_kv: int, D: int = 128, window=(-1, -1)) -> float:
    """4 * D FLOPs per visible (query, key) pair: cross-attention, grouped heads (which do not
    change the count) and key windows, whose hidden pairs are not counted."""
    return 4.0 * B * H * D * visible_pairs(S_q, S_kv, window)


def sage_prepare_bytes_ex(B: int, H: int, S_q: int, S_kv: int, H_kv: int, D: int = 128, rope_dim: int = 0,
                          smooth_k: bool = False) -> float:
    """sage_prepare_bytes for cross-attention / grouped-head shapes, plus the RMSNorm weights
    and RoPE tables of the fused transform (two [max(S_q, S_kv), rope_dim] BF16 tables) and,
    with K smoothing, one more read of K (its channel mean must be known before K is
    quantized) and the mean's write."""
    Spq, Spk = sage_padded_len(S_q), sage_padded_len(S_kv)
    read = 2.0 * (B * S_q * H * D + 3 * B * S_kv * H_kv * D)  # Q, K, V and V again
    write = (B * H * Spq * D + 2.0 * B * H_kv * Spk * D
             + 4.0 * (B * H * (Spq // 32) + B * H_kv * (Spk // 32) + B * H_kv * D))
    if rope_dim:
        read += 2.0 * 2 * max(S_q, S_kv) * rope_dim + 2.0 * 2 * D
    if smooth_k:
        read += 2.0 * B * S_kv * H_kv * D
        write += 4.0 * B * H_kv * D
    return read + write
