"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws random tensors,
rounds them to BF16 and picks which query rows a check samples.  Both the HIP
path and the CPU oracle consume exactly the BF16 bits it produces.

Workloads stand in for the DiT self-attention shapes the pages list
("Kernel acceleration: attention, compilation and fusion", section
"Attention: from O(N^2) memory to blocks", token-count table: FLUX 1024^2 has
4608 tokens, FLUX 2048^2 16896, Wan 2.1 720p 76112, HunyuanVideo 720p 119056;
24 x 128 and 40 x 128 channels) with randn inputs as in the randn benchmark of
"gfx1201_sage_prepare / gfx1201_sage_attention", section "Test Result".
The K bias of the FLUX-Sage and Wan workloads mimics DiT outlier channels: one
N(0, std = 2) value per (head, channel), shared by every token and batch.
"""
from dataclasses import dataclass

import numpy as np
import torch

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    seed: int
    k_bias_std: float = 0.0
    D: int = HEAD_DIM

    @property
    def scale(self) -> float:
        """Softmax scale float32(1 / sqrt(128))."""
        return float(np.float32(1.0 / np.sqrt(np.float64(self.D))))

    @property
    def flops(self) -> float:
        """Algorithmic attention FLOPs, 4 * B * H * S^2 * D."""
        return 4.0 * self.B * self.H * self.S * self.S * self.D


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 256, 1001),
    "flux1024": Workload("flux1024", 1, 24, 4608, 1002),
    "flux1024_kbias": Workload("flux1024_kbias", 1, 24, 4608, 1003, k_bias_std=2.0),
    "flux2048": Workload("flux2048", 1, 24, 16896, 1004),
    "wan720p": Workload("wan720p", 1, 40, 76112, 1005, k_bias_std=2.0),
    "hunyuan720p": Workload("hunyuan720p", 1, 24, 119056, 1006, k_bias_std=2.0),
}


def make_qkv(B, S, H, D=HEAD_DIM, seed=0, k_bias_std=0.0):
    """Q, K, V as contiguous CPU bfloat16 tensors [B, S, H, D].

    Draw order from one CPU generator: Q, K, V ~ N(0, 1), then the K bias
    k_bias_std * N(0, 1) of shape [H, D] (added to fp32 K); every tensor is
    rounded to BF16 (round to nearest even) last.
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((B, S, H, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, S, H, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, S, H, D), generator=g, dtype=torch.float32)
    if k_bias_std:
        bias = float(k_bias_std) * torch.randn((H, D), generator=g, dtype=torch.float32)
        k += bias
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def make_qkv_device(B, S, H, device, D=HEAD_DIM, seed=0, k_bias_std=0.0):
    """Same distribution as make_qkv, drawn on the GPU from a seeded device
    generator (fast at the video shapes).  The values differ from make_qkv's;
    the benchmark uses these only where no oracle comparison is made."""
    g = torch.Generator(device=device).manual_seed(int(seed))
    q = torch.randn((B, S, H, D), generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
    k = torch.randn((B, S, H, D), generator=g, dtype=torch.float32, device=device)
    v = torch.randn((B, S, H, D), generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
    if k_bias_std:
        bias = float(k_bias_std) * torch.randn((H, D), generator=g, dtype=torch.float32, device=device)
        k += bias
    return q, k.to(torch.bfloat16), v


def make_norm_weight(D=HEAD_DIM, seed=0):
    """A BF16 RMSNorm weight [D]: 1 + 0.25 * N(0, 1), seeded."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    return (1.0 + 0.25 * torch.randn(D, generator=g)).to(torch.bfloat16)


def make_rope_tables(S, rope_dim, base=10000.0):
    """BF16 cos/sin tables [S, rope_dim] of the rotate-half form: angle
    pos * base^(-i / (rope_dim / 2)) for i < rope_dim / 2, the two halves
    equal; computed in float64 and rounded to BF16 once."""
    half = rope_dim // 2
    inv = 1.0 / base ** (torch.arange(half, dtype=torch.float64) / half)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * inv[None, :]
    ang = torch.cat((ang, ang), dim=-1)
    return torch.cos(ang).to(torch.bfloat16), torch.sin(ang).to(torch.bfloat16)


def workload_qkv(w: Workload):
    return make_qkv(w.B, w.S, w.H, w.D, seed=w.seed, k_bias_std=w.k_bias_std)


def sample_rows(B, S, H, n=4096, seed=0):
    """Query rows to check, as an int64 array of (b, h, i) triples.

    When B * H * S <= n every row is returned.  Otherwise the last 32 rows of
    (b=0, h=0) and of (b=B-1, h=H-1) are always included (so the ragged query
    tail is checked) and the rest are drawn without replacement from a seeded
    permutation of all rows.
    """
    total = B * H * S
    if total <= n:
        b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(S), indexing="ij")
        return np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int64)
    forced = set()
    for (b, h) in ((0, 0), (B - 1, H - 1)):
        for i in range(max(0, S - 32), S):
            forced.add((b * H + h) * S + i)
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    flat = list(sorted(forced))
    need = n - len(flat)
    perm = torch.randperm(total, generator=g)
    picked = []
    for x in perm[: need + len(forced)].tolist():
        if x not in forced:
            picked.append(x)
        if len(picked) == need:
            break
    flat = np.array(sorted(flat + picked), dtype=np.int64)
    b = flat // (H * S)
    h = (flat // S) % H
    i = flat % S
    return np.stack([b, h, i], axis=1)
