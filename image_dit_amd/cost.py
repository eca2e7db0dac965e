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
