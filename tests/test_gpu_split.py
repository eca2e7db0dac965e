"""GPU checks of attn_fwd_bf16_ws, the BF16 attention whose last, partial round of query
tiles is split over every compute unit ("Kernel acceleration: attention, compilation and
fusion", section "Attention: from O(N^2) memory to blocks": the pieces of a query tile are
merged with the same running-max rescaling the blocked form uses).

  * the split is taken for these shapes (the workspace size is not 0) and not for shapes with
    fewer than three whole rounds of query tiles (FLUX-1024 among them) or a full last round;
  * against exact fp64 attention: the BF16 gates (max abs <= 1e-2, cosine >= 0.99999);
  * against attn_fwd_bf16_ex (no split): within 2e-3, with the same error against the exact
    result (P is rounded to BF16 relative to each piece's own running max);
  * run-to-run bitwise deterministic, also when one workspace serves consecutive calls;
  * shapes that are not split give exactly attn_fwd_bf16_ex's output.
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


def qkv(B, S_q, S_kv, H, H_kv, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(B, S_q, H, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(B, S_kv, H_kv, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(B, S_kv, H_kv, 128, generator=g).to(torch.bfloat16)
    return q, k, v


SPLIT = [  # (B, S_q, S_kv, H, H_kv, seed): 864 query tiles = three whole rounds of 256 + 96
    (1, 4608, 4608, 48, 48, 71),   # 72 key tiles per query tile
    (2, 4600, 4600, 24, 24, 72),   # ragged query and key tails
    (2, 4608, 1000, 24, 6, 73),    # cross-attention + grouped heads: 16 key tiles per query
                                   # tile, each tail tile spread over about six workgroups
]


@pytest.mark.parametrize("shape", SPLIT, ids=lambda s: "B%d-q%d-kv%d-h%d-hkv%d" % s[:5])
def test_split_matches_oracle_and_unsplit(shape):
    B, S_q, S_kv, H, H_kv, seed = shape
    log("[split %s]" % (shape,))
    need = ia.bf16_workspace_size(B, S_q, S_kv, H, H_kv)
    assert need > 0, "the split is not taken for this shape on this device"
    qc, kc, vc = qkv(B, S_q, S_kv, H, H_kv, seed)
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    o1 = ia.attn_fwd_bf16_ws(q, k, v, SCALE, workspace=ws)
    o2 = ia.attn_fwd_bf16_ws(q, k, v, SCALE, workspace=ws)  # same workspace, next call
    ref_gpu = ia.attn_fwd_bf16_ex(q, k, v, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "not deterministic"
    assert not torch.isnan(o1.float()).any()
    # P is rounded to BF16 relative to each piece's own running max, so the two differ by the
    # rounding of P (about 1e-4 here), not only by the final BF16 rounding
    d = (o1.float() - ref_gpu.float()).abs().max().item()
    assert d <= 2e-3, "max |split - unsplit| = %g" % d
    rows = synth.sample_rows(B, S_q, H, n=2048, seed=seed + 1)
    ref = oracle.attn_rows_ex(qc, kc, vc, SCALE, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    rel = {}
    for name, o in (("split", o1), ("unsplit", ref_gpu)):
        got = o[idx[:, 0], idx[:, 2], idx[:, 1]].float().cpu().numpy().astype(np.float64)
        cos = float((got * ref).sum() / np.linalg.norm(got) / np.linalg.norm(ref))
        mx = float(np.max(np.abs(got - ref)))
        rel[name] = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        log("  %s: max abs %.2e cos %.7f relL2 %.5f" % (name, mx, cos, rel[name]))
        assert mx <= 1e-2 and cos >= 0.99999, (name, mx, cos)
    assert rel["split"] <= 1.05 * rel["unsplit"] + 1e-4, rel


@pytest.mark.parametrize("shape", [(1, 4096, 4096, 16, 16), (1, 300, 300, 2, 2), (1, 2000, 2000, 64, 8),
                                   (1, 4608, 4608, 24, 24)],
                         ids=lambda s: "B%d-q%d-kv%d-h%d-hkv%d" % s)
def test_unsplit_shapes_equal_ex(shape):
    B, S_q, S_kv, H, H_kv = shape
    log("[unsplit %s]" % (shape,))
    assert ia.bf16_workspace_size(B, S_q, S_kv, H, H_kv) == 0
    q, k, v = (t.cuda() for t in qkv(B, S_q, S_kv, H, H_kv, 81))
    a = ia.attn_fwd_bf16_ws(q, k, v, SCALE)
    b = ia.attn_fwd_bf16_ex(q, k, v, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_windowed_calls_are_not_split():
    assert ia.bf16_workspace_size(1, 4608, 4608, 24, 24, (-1, 0)) == 0
    assert ia.bf16_workspace_size(1, 4608, 4608, 24, 24, (256, 256)) == 0


def test_split_on_another_stream_equals_the_current_stream():
    # Both split-tail entry points on a second stream with the binding's own workspace: its
    # zero fill runs on the current stream and the second stream waits for it, so every call
    # gives the output of the current-stream call bit for bit.
    B, S, H = 1, 4608, 48
    log("[split on another stream B=%d S=%d H=%d]" % (B, S, H))
    assert ia.bf16_workspace_size(B, S, S, H, H) > 0
    g = torch.Generator().manual_seed(95)
    q, k, v = (torch.randn(B, S, H, 128, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    prepared = ia.sage_prepare_ex(q, k, v, SCALE)
    ref_b = ia.attn_fwd_bf16_ws(q, k, v, SCALE)
    ref_s = ia.sage_attn_fwd_ws(prepared, S, S, H, H, SCALE)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = [(ia.attn_fwd_bf16_ws(q, k, v, SCALE, stream=side),
             ia.sage_attn_fwd_ws(prepared, S, S, H, H, SCALE, stream=side)) for _ in range(3)]
    torch.cuda.synchronize()
    for ob, os_ in outs:
        assert torch.equal(ob.view(torch.int16), ref_b.view(torch.int16))
        assert torch.equal(os_.view(torch.int16), ref_s.view(torch.int16))
