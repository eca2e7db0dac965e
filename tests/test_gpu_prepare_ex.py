"""GPU checks of the prepare stage's options through the C ABI (bitwise).

  * qk_norm_rope_bf16 (RMSNorm + rotate-half RoPE, BF16 rounding after every
    eager step) against the CPU oracle, every rope_dim of the page
    ("gfx1201_sage_prepare / gfx1201_sage_attention", first commit and
    "Technical Details": rope_dim 32/64/96/128);
  * sage_prepare_ex with the transform fused equals qk_norm_rope_bf16 followed
    by sage_prepare, bit for bit (the page's "fused == unfused bitwise"), and
    both equal the oracle;
  * K smoothing ("Kernel acceleration: attention, compilation and fusion",
    section "SageAttention: quantizing attention too"): the channel mean and
    the codes bitwise against the oracle, and the attention it feeds within the
    Sage gates with a smaller error than without smoothing;
  * cross-attention and grouped-query shapes of the prepare stage.
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
EPS = 1e-6
NAMES = ("q_i8", "q_scale", "k_i8", "k_scale", "v_fp8", "v_scale", "k_mean")


def log(msg):
    print(msg, flush=True)


def same_bits(got, ref):
    g = got.cpu().numpy() if isinstance(got, torch.Tensor) else got
    r = ref.cpu().numpy() if isinstance(ref, torch.Tensor) else ref
    if g.dtype == np.float32:
        g, r = g.view(np.uint32), r.view(np.uint32)
    if g.dtype in (np.int16,) or str(g.dtype) == "bfloat16":
        g, r = g.view(np.uint16), r.view(np.uint16)
    return g.shape == r.shape and np.array_equal(g, r)


def bits16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def assert_prepared_equal(got, ref, what):
    for name, g, r in zip(NAMES, got, ref):
        g = g.cpu().numpy() if isinstance(g, torch.Tensor) else g
        r = r.cpu().numpy() if isinstance(r, torch.Tensor) else r
        assert g.shape == r.shape, (what, name, g.shape, r.shape)
        if g.dtype == np.float32:
            bad = np.count_nonzero(g.view(np.uint32) != r.view(np.uint32))
        else:
            bad = np.count_nonzero(g != r)
        assert bad == 0, "%s: %s differs in %d of %d" % (what, name, bad, g.size)


def transform_inputs(S, rope_dim, norm, seed):
    wq = synth.make_norm_weight(seed=seed) if norm else None
    wk = synth.make_norm_weight(seed=seed + 1) if norm else None
    cos, sin = synth.make_rope_tables(S, rope_dim) if rope_dim else (None, None)
    return wq, wk, cos, sin


def cuda(*ts):
    return [t.cuda() if t is not None else None for t in ts]


@pytest.mark.parametrize("rope_dim,norm", [(r, n) for n in (True, False) for r in (0, 32, 64, 96, 128)
                                           if n or r])  # neither: the identity
def test_qk_norm_rope_matches_oracle(rope_dim, norm):
    B, S, H = 2, 300, 3
    log("[xform rope_dim=%d norm=%d]" % (rope_dim, norm))
    x, _, _ = synth.make_qkv(B, S, H, seed=400 + rope_dim, k_bias_std=0.0)
    x = (3 * x.float()).to(torch.bfloat16)
    w, _, cos, sin = transform_inputs(S, rope_dim, norm, seed=rope_dim)
    ref = oracle.qk_norm_rope(x, w, EPS, cos, sin, rope_dim)
    xd, wd, cd, sd = cuda(x, w, cos, sin)
    got = ia.qk_norm_rope_bf16(xd, wd, EPS, cd, sd, rope_dim)
    assert np.array_equal(bits16(got), ref)
    # in place gives the same bits
    ia.qk_norm_rope_bf16(xd, wd, EPS, cd, sd, rope_dim, out=xd)
    assert np.array_equal(bits16(xd), ref)


@pytest.mark.parametrize("rope_dim,norm,smooth", [(128, True, False), (64, True, True), (96, False, False),
                                                  (32, True, False), (0, True, True), (0, False, True)])
def test_fused_prepare_equals_unfused_and_oracle(rope_dim, norm, smooth):
    B, S, H = 1, 333, 4
    log("[fused rope_dim=%d norm=%d smooth=%d]" % (rope_dim, norm, smooth))
    q, k, v = synth.make_qkv(B, S, H, seed=500 + rope_dim + norm, k_bias_std=2.0)
    wq, wk, cos, sin = transform_inputs(S, rope_dim, norm, seed=7)
    ref = oracle.sage_prepare_ex(q, k, v, SCALE, wq, wk, EPS, cos, sin, rope_dim, smooth_k=smooth)
    qd, kd, vd, wqd, wkd, cd, sd = cuda(q, k, v, wq, wk, cos, sin)
    fused = ia.sage_prepare_ex(qd, kd, vd, SCALE, wqd, wkd, EPS, cd, sd, rope_dim, smooth_k=smooth)
    assert_prepared_equal(fused, ref, "fused vs oracle")
    qt = ia.qk_norm_rope_bf16(qd, wqd, EPS, cd, sd, rope_dim) if (norm or rope_dim) else qd
    kt = ia.qk_norm_rope_bf16(kd, wkd, EPS, cd, sd, rope_dim) if (norm or rope_dim) else kd
    unfused = ia.sage_prepare_ex(qt, kt, vd, SCALE, smooth_k=smooth)
    assert_prepared_equal(fused, unfused, "fused vs unfused")


def sage_metrics(out, ref):
    got = out.float().cpu().numpy().astype(np.float64).reshape(-1, 128)
    r = ref.reshape(-1, 128)
    cos = float(np.sum(got * r) / (np.linalg.norm(got) * np.linalg.norm(r)))
    rel = float(np.linalg.norm(got - r) / np.linalg.norm(r))
    return cos, rel


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wname", ["flux1024_kbias", "wan720p"])
def test_smoothing_bitwise_and_more_accurate(wname):
    w = synth.WORKLOADS[wname]
    log("[smooth %s] inputs" % wname)
    q, k, v = synth.workload_qkv(w)
    ref = oracle.sage_prepare_ex(q, k, v, w.scale, smooth_k=True)
    qd, kd, vd = cuda(q, k, v)
    log("[smooth %s] sage_prepare_ex" % wname)
    got = ia.sage_prepare_ex(qd, kd, vd, w.scale, smooth_k=True)
    torch.cuda.synchronize()
    assert_prepared_equal(got, ref, "smoothed prepare")
    rows = synth.sample_rows(w.B, w.S, w.H, n=1024, seed=w.seed + 1)
    exact = oracle.attn_rows(q, k, v, w.scale, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    outs = {}
    for smooth in (False, True):
        prep = got[:6] if smooth else ia.sage_prepare(qd, kd, vd, w.scale)
        o = ia.sage_attn_fwd(prep, w.S, w.H, w.scale)
        outs[smooth] = sage_metrics(o[idx[:, 0], idx[:, 2], idx[:, 1]], exact)
    log("[smooth %s] plain cos %.6f rel %.5f; smoothed cos %.6f rel %.5f" % (wname, *outs[False], *outs[True]))
    cos, rel = outs[True]
    assert cos >= 0.998 and rel <= 5e-2
    assert rel < outs[False][1]


@pytest.mark.parametrize("S_q,S_kv,H,H_kv", [(300, 77, 4, 2), (64, 1000, 6, 1), (513, 512, 2, 2)])
def test_prepare_cross_and_grouped_shapes(S_q, S_kv, H, H_kv):
    B = 2
    log("[cross prep S_q=%d S_kv=%d H=%d H_kv=%d]" % (S_q, S_kv, H, H_kv))
    g = torch.Generator().manual_seed(S_q + S_kv)
    q = torch.randn((B, S_q, H, 128), generator=g).to(torch.bfloat16)
    k = (torch.randn((B, S_kv, H_kv, 128), generator=g) + 2 * torch.randn((H_kv, 128), generator=g)).to(torch.bfloat16)
    v = torch.randn((B, S_kv, H_kv, 128), generator=g).to(torch.bfloat16)
    wq, wk, cos, sin = transform_inputs(max(S_q, S_kv), 64, True, seed=3)
    ref = oracle.sage_prepare_ex(q, k, v, SCALE, wq, wk, EPS, cos, sin, 64, smooth_k=True)
    got = ia.sage_prepare_ex(*cuda(q, k, v), SCALE, *cuda(wq, wk), EPS, *cuda(cos, sin), 64, smooth_k=True)
    assert_prepared_equal(got, ref, "cross prepare")
