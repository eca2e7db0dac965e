"""sage_prepare_ex_noalloc through the C ABI: K smoothing from the library's
static device scratch instead of a caller workspace gives, bit for bit, what
sage_prepare_ex gives with one.  Two calls in a row on one device, the second
smaller, so the second runs over the scratch the first left behind."""
import math

import numpy as np
import pytest
import torch

import image_dit_amd as ia
from image_dit_amd import synth

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / math.sqrt(128)))
NAMES = ("q_i8", "q_scale", "k_i8", "k_scale", "v_fp8", "v_scale", "k_mean")


def log(msg):
    print(msg, flush=True)


def same(got, ref, what):
    for name, g, r in zip(NAMES, got, ref):
        g, r = g.cpu(), r.cpu()
        assert g.shape == r.shape and g.dtype == r.dtype, (what, name)
        if g.dtype == torch.float32:
            g, r = g.view(torch.int32), r.view(torch.int32)
        bad = int((g != r).sum())
        assert bad == 0, "%s: %s differs in %d of %d" % (what, name, bad, g.numel())


def fresh_out(B, S_q, S_kv, H, H_kv):
    """Output buffers filled with a value no result takes everywhere."""
    S_qp, S_kp = ia.sage_padded_len(S_q), ia.sage_padded_len(S_kv)
    out = (torch.full((B, H, S_qp, 128), 7, dtype=torch.int8, device="cuda"),
           torch.full((B, H, S_qp // 32), 7.0, dtype=torch.float32, device="cuda"),
           torch.full((B, H_kv, S_kp, 128), 7, dtype=torch.int8, device="cuda"),
           torch.full((B, H_kv, S_kp // 32), 7.0, dtype=torch.float32, device="cuda"),
           torch.full((B, H_kv, 128, S_kp), 7, dtype=torch.uint8, device="cuda"),
           torch.full((B, H_kv, 128), 7.0, dtype=torch.float32, device="cuda"))
    return out


CASES = [  # (B, S_q, S_kv, H, H_kv, norm, rope_dim, kbias, seed); each smaller than the one before
    (2, 1000, 1300, 6, 3, True, 64, 2.0, 11),
    (1, 300, 333, 2, 1, True, 128, 1.0, 12),
    (1, 70, 45, 1, 1, False, 0, 0.5, 13),
]


@pytest.mark.parametrize("smooth", [True, False])
def test_noalloc_matches_workspace_entry(smooth):
    for B, S_q, S_kv, H, H_kv, norm, rope_dim, kbias, seed in CASES:
        log("[noalloc smooth=%d B=%d S_q=%d S_kv=%d H=%d H_kv=%d rope=%d]"
            % (smooth, B, S_q, S_kv, H, H_kv, rope_dim))
        need = ia.sage_workspace_size(B, S_kv, H_kv)
        assert need <= ia.STATIC_SCRATCH_BYTES
        g = torch.Generator(device="cuda").manual_seed(seed)
        q = torch.randn(B, S_q, H, 128, generator=g, device="cuda").to(torch.bfloat16)
        k = (torch.randn(B, S_kv, H_kv, 128, generator=g, device="cuda")
             + kbias * torch.randn(1, 1, H_kv, 128, generator=g, device="cuda")).to(torch.bfloat16)
        v = torch.randn(B, S_kv, H_kv, 128, generator=g, device="cuda").to(torch.bfloat16)
        xf = {}
        if norm:
            xf["q_norm_w"] = synth.make_norm_weight(seed=seed).cuda()
            xf["k_norm_w"] = synth.make_norm_weight(seed=seed + 1).cuda()
        if rope_dim:
            cos, sin = synth.make_rope_tables(max(S_q, S_kv), rope_dim)
            xf.update(rope_cos=cos.cuda(), rope_sin=sin.cuda(), rope_dim=rope_dim)
        ref = ia.sage_prepare_ex(q, k, v, SCALE, smooth_k=smooth, **xf)
        out = fresh_out(B, S_q, S_kv, H, H_kv)
        k_mean = torch.full((B, H_kv, 128), 7.0, device="cuda") if smooth else None
        got = ia.sage_prepare_ex_noalloc(q, k, v, SCALE, out=out, k_mean=k_mean, **xf)
        torch.cuda.synchronize()
        assert len(got) == len(ref)
        same(got, ref, "noalloc vs workspace")
        # the outputs are usable: Sage attention from them equals the one from the reference
        o_ref = ia.sage_attn_fwd_ex(ref[:6], S_q, S_kv, H, H_kv, SCALE)
        o_got = ia.sage_attn_fwd_ex(got[:6], S_q, S_kv, H, H_kv, SCALE)
        torch.cuda.synchronize()
        assert torch.equal(o_ref.view(torch.int16), o_got.view(torch.int16))
