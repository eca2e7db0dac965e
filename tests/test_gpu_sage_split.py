"""GPU checks of sage_attn_fwd_ws, the Sage attention whose last, partial round of query tiles
is split over every compute unit ("Kernel acceleration: attention, compilation and fusion",
section "Attention: from O(N^2) memory to blocks": the pieces of a query tile are merged with
the same running-max rescaling the blocked form uses; the quantized operands are those of
"gfx1201_sage_prepare / gfx1201_sage_attention", "Technical Details").

  * the split is taken for these shapes (the workspace size is not 0), with the same plan as
    the BF16 path, and not for shapes with fewer than three whole rounds of query tiles;
  * against exact fp64 attention on the BF16 inputs: the Sage gates (cosine >= 0.998,
    relative L2 <= 5e-2), with an error no larger than sage_attn_fwd_ex's (P is rounded to FP8
    relative to each piece's own running max, so the two outputs differ by that rounding); the
    same gates against attention of the oracle's quantized operands;
  * run-to-run bitwise deterministic, also when one workspace serves consecutive calls;
  * shapes that are not split give exactly sage_attn_fwd_ex's output.
"""
import math

import numpy as np
import pytest
import torch

import image_dit_amd as ia
import oracle
from image_dit_amd import synth

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / math.sqrt(128)))


def log(msg):
    print(msg, flush=True)


def qkv(B, S_q, S_kv, H, H_kv, seed, k_bias_std=0.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(B, S_q, H, 128, generator=g)
    k = torch.randn(B, S_kv, H_kv, 128, generator=g)
    v = torch.randn(B, S_kv, H_kv, 128, generator=g)
    if k_bias_std:
        k = k + k_bias_std * torch.randn(H_kv, 128, generator=g)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


SPLIT = [  # (B, S_q, S_kv, H, H_kv, K bias std, seed): 864 query tiles = three whole rounds of 256 + 96
    (1, 4608, 4608, 48, 48, 2.0, 91),   # 72 key tiles per query tile, DiT-like K outlier channels
    (2, 4600, 4600, 24, 24, 0.0, 92),   # ragged query and key tails
    (2, 4608, 1000, 24, 6, 0.0, 93),    # cross-attention + grouped heads: 16 key tiles per query tile
]


@pytest.mark.parametrize("shape", SPLIT, ids=lambda s: "B%d-q%d-kv%d-h%d-hkv%d" % s[:5])
def test_sage_split_matches_oracle_and_unsplit(shape):
    B, S_q, S_kv, H, H_kv, kb, seed = shape
    log("[sage split %s]" % (shape,))
    need = ia.sage_attn_workspace_size(B, S_q, S_kv, H, H_kv)
    assert need > 0, "the split is not taken for this shape on this device"
    assert need == ia.bf16_workspace_size(B, S_q, S_kv, H, H_kv)
    qc, kc, vc = qkv(B, S_q, S_kv, H, H_kv, seed, kb)
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    prepared = ia.sage_prepare_ex(q, k, v, SCALE)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    o1 = ia.sage_attn_fwd_ws(prepared, S_q, S_kv, H, H_kv, SCALE, workspace=ws)
    o2 = ia.sage_attn_fwd_ws(prepared, S_q, S_kv, H, H_kv, SCALE, workspace=ws)  # same workspace
    ref_gpu = ia.sage_attn_fwd_ex(prepared, S_q, S_kv, H, H_kv, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "not deterministic"
    assert not torch.isnan(o1.float()).any()
    rows = synth.sample_rows(B, S_q, H, n=2048, seed=seed + 1)
    ref = oracle.attn_rows_ex(qc, kc, vc, SCALE, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    rel = {}
    for name, o in (("split", o1), ("unsplit", ref_gpu)):
        got = o[idx[:, 0], idx[:, 2], idx[:, 1]].float().cpu().numpy().astype(np.float64)
        cos = float((got * ref).sum() / np.linalg.norm(got) / np.linalg.norm(ref))
        rel[name] = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        log("  %s: cos %.5f relL2 %.4f max abs %.2e" % (name, cos, rel[name], float(np.max(np.abs(got - ref)))))
        assert cos >= 0.998 and rel[name] <= 5e-2, (name, cos, rel[name])
    assert rel["split"] <= 1.05 * rel["unsplit"] + 1e-3, rel
    # the kernel's own error: against attention of the oracle's quantized operands
    ref_q = oracle.sage_attn_rows_ex(oracle.sage_prepare_ex(qc, kc, vc, SCALE), S_q, S_kv, (-1, -1), rows)
    got = o1[idx[:, 0], idx[:, 2], idx[:, 1]].float().cpu().numpy().astype(np.float64)
    cos = float((got * ref_q).sum() / np.linalg.norm(got) / np.linalg.norm(ref_q))
    rel_q = float(np.linalg.norm(got - ref_q) / np.linalg.norm(ref_q))
    log("  split vs quantized operands: cos %.5f relL2 %.4f" % (cos, rel_q))
    assert cos >= 0.998 and rel_q <= 5e-2, (cos, rel_q)


@pytest.mark.parametrize("shape", [(1, 4096, 4096, 16, 16), (1, 300, 300, 2, 2), (1, 2000, 2000, 64, 8),
                                   (1, 4608, 4608, 24, 24)],
                         ids=lambda s: "B%d-q%d-kv%d-h%d-hkv%d" % s)
def test_sage_unsplit_shapes_equal_ex(shape):
    B, S_q, S_kv, H, H_kv = shape
    log("[sage unsplit %s]" % (shape,))
    assert ia.sage_attn_workspace_size(B, S_q, S_kv, H, H_kv) == 0
    q, k, v = (t.cuda() for t in qkv(B, S_q, S_kv, H, H_kv, 94))
    prepared = ia.sage_prepare_ex(q, k, v, SCALE)
    a = ia.sage_attn_fwd_ws(prepared, S_q, S_kv, H, H_kv, SCALE)
    b = ia.sage_attn_fwd_ex(prepared, S_q, S_kv, H, H_kv, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_sage_windowed_calls_are_not_split():
    assert ia.sage_attn_workspace_size(1, 4608, 4608, 24, 24, (-1, 0)) == 0
    assert ia.sage_attn_workspace_size(1, 4608, 4608, 24, 24, (256, 256)) == 0
