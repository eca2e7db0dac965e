"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Exact attention ("Kernel acceleration: attention, compilation and fusion",
section "Attention: from O(N^2) memory to blocks") is pinned by invariants of
softmax attention, closed forms at S = 1 and S = 2, the page's own blocked
form, and PyTorch's scaled_dot_product_attention in float64 as an independent
library routine.  The quantizer ("gfx1201_sage_prepare /
gfx1201_sage_attention", section "Technical Details") is pinned by hand-made
blocks with known codes, the OCP E4M3 value table and torch's float8_e4m3fn
conversion.  Attention of the quantized operands (same page, commit text of the
attention op) is pinned to exact attention on inputs the quantizer represents
exactly, and by its closed forms at one key and at equal scores.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from image_dit_amd import synth

SCALE = float(np.float32(1.0 / math.sqrt(128.0)))


def bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def rand_qkv(B, S, H, D=128, seed=0):
    return synth.make_qkv(B, S, H, D, seed=seed)


def f64(x):
    return x.to(torch.float64).numpy()


# --------------------------------------------------------------------------
# exact attention
# --------------------------------------------------------------------------

def test_softmax_rows_sum_to_one():
    q, k, _ = rand_qkv(1, 97, 2, seed=1)
    for (h, i) in [(0, 0), (1, 50), (0, 96)]:
        p = oracle.softmax_row(q, k, SCALE, 0, h, i)
        assert p.min() >= 0.0
        assert abs(p.sum() - 1.0) < 1e-12


def test_constant_v_returns_v():
    B, S, H, D = 2, 65, 3, 128
    q, k, _ = rand_qkv(B, S, H, D, seed=2)
    u = torch.randn((1, 1, H, D), generator=torch.Generator().manual_seed(3))
    v = bf16(u.expand(B, S, H, D).contiguous())
    out = oracle.attn_rows(q, k, v, SCALE)
    ref = np.broadcast_to(f64(v[:, :1]), out.shape)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_identical_keys_give_mean_of_v():
    B, S, H, D = 1, 80, 2, 128
    q, _, v = rand_qkv(B, S, H, D, seed=4)
    k1 = torch.randn((B, 1, H, D), generator=torch.Generator().manual_seed(5))
    k = bf16(k1.expand(B, S, H, D).contiguous())
    out = oracle.attn_rows(q, k, v, SCALE)
    mean_v = f64(v).mean(axis=1, keepdims=True)
    assert np.max(np.abs(out - mean_v)) < 1e-12


def test_per_row_shift_of_all_keys_is_a_noop():
    # k_j + w for one vector w and every key j shifts each score row by the
    # constant q.w * scale, which the softmax removes.  Values are multiples
    # of 1/16 below 8 in magnitude, so k + w is exact in BF16.
    B, S, H, D = 1, 70, 2, 128
    g = torch.Generator().manual_seed(6)
    q = bf16(torch.randint(-32, 33, (B, S, H, D), generator=g) / 16.0)
    k = bf16(torch.randint(-64, 65, (B, S, H, D), generator=g) / 16.0)
    w = torch.randint(-64, 65, (1, 1, H, D), generator=g) / 16.0
    v = bf16(torch.randn((B, S, H, D), generator=g))
    k_shift = bf16(k.float() + w)
    assert torch.equal(k_shift.float(), k.float() + w)  # exact
    a = oracle.attn_rows(q, k, v, SCALE)
    b = oracle.attn_rows(q, k_shift, v, SCALE)
    assert np.max(np.abs(a - b)) < 1e-12


def test_token_permutations():
    B, S, H, D = 1, 90, 2, 128
    q, k, v = rand_qkv(B, S, H, D, seed=7)
    base = oracle.attn_rows(q, k, v, SCALE)
    g = torch.Generator().manual_seed(8)
    pq = torch.randperm(S, generator=g)
    out_q = oracle.attn_rows(q[:, pq].contiguous(), k, v, SCALE)
    assert np.max(np.abs(out_q - base[:, pq.numpy()])) < 1e-13
    pk = torch.randperm(S, generator=g)
    out_kv = oracle.attn_rows(q, k[:, pk].contiguous(), v[:, pk].contiguous(), SCALE)
    assert np.max(np.abs(out_kv - base)) < 1e-12
    # token order reversal of K/V together, as in the noise-floor run
    rev = torch.arange(S - 1, -1, -1)
    out_rev = oracle.attn_rows(q, k[:, rev].contiguous(), v[:, rev].contiguous(), SCALE)
    assert np.max(np.abs(out_rev - base)) < 1e-12


def test_single_key_returns_its_value():
    q, k, v = rand_qkv(2, 1, 3, seed=9)
    out = oracle.attn_rows(q, k, v, SCALE)
    assert np.array_equal(out, f64(v))


def test_two_keys_closed_form():
    # o = sigmoid(d) v0 + sigmoid(-d) v1 with d = s0 - s1.
    B, S, H, D = 1, 2, 2, 128
    q, k, v = rand_qkv(B, S, H, D, seed=10)
    out = oracle.attn_rows(q, k, v, SCALE)
    qd, kd, vd = f64(q), f64(k), f64(v)
    for i in range(S):
        for h in range(H):
            s0 = float(np.dot(qd[0, i, h], kd[0, 0, h])) * SCALE
            s1 = float(np.dot(qd[0, i, h], kd[0, 1, h])) * SCALE
            dlt = s0 - s1
            sig = 1.0 / (1.0 + math.exp(-dlt))
            ref = sig * vd[0, 0, h] + (1.0 - sig) * vd[0, 1, h]
            assert np.max(np.abs(out[0, i, h] - ref)) < 1e-13


@pytest.mark.parametrize("bq,bk", [(64, 64), (16, 256), (33, 7), (256, 16)])
def test_blocked_form_matches_naive(bq, bk):
    B, S, H, D = 2, 123, 2, 128
    q, k, v = rand_qkv(B, S, H, D, seed=11)
    a = oracle.attn_rows(q, k, v, SCALE)
    b = oracle.attn_blocked(q, k, v, SCALE, bq=bq, bk=bk)
    assert np.max(np.abs(a - b)) < 1e-12


def test_matches_torch_sdpa_float64():
    B, S, H, D = 2, 150, 3, 128
    q, k, v = rand_qkv(B, S, H, D, seed=12)
    out = oracle.attn_rows(q, k, v, SCALE)
    t = lambda x: x.to(torch.float64).permute(0, 2, 1, 3).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=SCALE)
    ref = ref.permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_sampled_rows_agree_with_full():
    B, S, H, D = 2, 100, 3, 128
    q, k, v = rand_qkv(B, S, H, D, seed=13)
    full = oracle.attn_rows(q, k, v, SCALE)
    rows = synth.sample_rows(B, S, H, n=200, seed=14)
    part = oracle.attn_rows(q, k, v, SCALE, rows=rows)
    assert np.array_equal(part, full[rows[:, 0], rows[:, 2], rows[:, 1]])


def test_scale_enters_once():
    # Doubling the scale equals doubling Q when Q doubles exactly.
    q, k, v = rand_qkv(1, 40, 1, seed=15)
    a = oracle.attn_rows(q, k, v, 2 * SCALE)
    b = oracle.attn_rows(bf16(q.float() * 2), k, v, SCALE)
    assert np.max(np.abs(a - b)) < 1e-12


def test_row_sampler_forces_tail_rows():
    rows = synth.sample_rows(1, 76112, 40, n=4096, seed=1006)
    assert rows.shape == (4096, 3)
    assert len({tuple(r) for r in rows.tolist()}) == 4096
    tail = {(0, 0, i) for i in range(76112 - 32, 76112)} | {(0, 39, i) for i in range(76112 - 32, 76112)}
    assert tail <= {tuple(r) for r in rows.tolist()}


# --------------------------------------------------------------------------
# quantizer
# --------------------------------------------------------------------------

E4M3_TABLE = [  # (value, code) from the OCP E4M3 definition: bias 7, 3 mantissa bits, max 448
    (448.0, 0x7E), (1.0, 0x38), (2.0 ** -9, 0x01), (2.0 ** -6, 0x08), (-1.0, 0xB8),
    (1.0625, 0x38), (1.1875, 0x3A), (464.0, 0x7E), (240.0, 0x77), (0.0, 0x00),
    (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (-3 * 2.0 ** -10, 0x82), (256.0, 0x78),
]


@pytest.mark.parametrize("x,code", E4M3_TABLE)
def test_e4m3_known_codes(x, code):
    assert oracle.e4m3_encode(x) == code


def test_e4m3_decode_table():
    vals = [oracle.e4m3_decode(c) for c in range(127)]
    assert vals[0] == 0.0 and vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6 and vals[126] == 448.0
    assert all(a < b for a, b in zip(vals, vals[1:]))  # strictly increasing
    assert math.isnan(oracle.e4m3_decode(0x7F))
    for c in range(127):
        assert oracle.e4m3_encode(vals[c]) == c
        assert oracle.e4m3_encode(-vals[c]) == 0x80 | c


def test_e4m3_matches_torch_float8_e4m3fn():
    vals = np.array([oracle.e4m3_decode(c) for c in range(127)])
    mids = (vals[:-1] + vals[1:]) / 2
    xs = [vals, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
          np.nextafter(mids.astype(np.float32), np.float32(1000))]
    allbf = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float().numpy()
    xs.append(allbf[np.isfinite(allbf) & (np.abs(allbf) <= 448)])
    xs.append(np.random.default_rng(0).uniform(-448, 448, 20000))
    x = np.concatenate([np.concatenate(xs), -np.concatenate(xs)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def _put_block(values, S=32, H=1, D=128, h=0, rows=None):
    x = torch.zeros((1, S, H, D), dtype=torch.float32)
    flat = x[0, :32, h].reshape(-1)
    flat[: len(values)] = torch.tensor(values, dtype=torch.float32)
    x[0, :32, h] = flat.reshape(32, D)
    return bf16(x)


def test_quant_round_half_even_at_unit_scale():
    vals = [127.0, 2.5, 3.5, -0.5, -1.5, 0.5, -2.5, 1.25, -126.5]
    codes, scales = oracle.quant_qk(_put_block(vals), 1.0)
    assert scales[0, 0, 0] == np.float32(1.0)
    assert scales.shape == (1, 1, 8)  # S_pad = 256
    assert list(codes[0, 0, 0, :9]) == [127, 2, 4, 0, -2, 0, -2, 1, -126]
    assert not codes[0, 0, 0, 9:].any() and not codes[0, 0, 1:].any()
    assert np.all(scales[0, 0, 1:] == 0)


def test_quant_absmax_maps_to_127_and_error_bound():
    q, k, _ = rand_qkv(2, 300, 3, seed=16)
    for x, mult in ((k, 1.0), (q, oracle.q_multiplier(SCALE))):
        codes, scales = oracle.quant_qk(x, mult)
        S_pad = codes.shape[2]
        assert S_pad == 512
        y = (x.float() * np.float32(mult)).numpy().astype(np.float32)  # [B,S,H,D]
        y = np.transpose(y, (0, 2, 1, 3))  # [B,H,S,D]
        for b in range(2):
            for h in range(3):
                for blk in range(S_pad // 32):
                    c = codes[b, h, blk * 32:(blk + 1) * 32].astype(np.float64)
                    s = float(scales[b, h, blk])
                    yb = y[b, h, blk * 32:min(blk * 32 + 32, 300)]
                    if yb.shape[0] == 0:
                        assert s == 0.0 and not c.any()
                        continue
                    amax = np.abs(yb).max()
                    assert s == np.float32(np.float32(amax) / np.float32(127.0))
                    arg = np.unravel_index(np.argmax(np.abs(yb)), yb.shape)
                    assert abs(c[arg]) == 127
                    err = np.abs(yb - c[: yb.shape[0]] * s)
                    assert err.max() <= s / 2 * (1 + 1e-5)
                    assert not c[yb.shape[0]:].any()  # pad rows


def test_quant_zero_block():
    x = bf16(torch.zeros((1, 64, 1, 128)))
    codes, scales = oracle.quant_qk(x, 1.0)
    assert not codes.any() and not scales.any()
    vcodes, vscales = oracle.quant_v(x)
    assert not vcodes.any() and not vscales.any()


def test_q_multiplier_is_scale_times_log2e():
    c = oracle.q_multiplier(SCALE)
    # float32(1/sqrt(128)) / ln 2 rounded once to fp32 (an independent route)
    assert np.float32(c) == np.float32(np.float64(np.float32(1 / math.sqrt(128))) / math.log(2.0))
    assert np.float32(c).view(np.uint32) == 0x3E0293EE


def test_quant_matches_torch_vectorized():
    q, k, _ = rand_qkv(1, 200, 2, seed=17)
    for x, mult in ((k, 1.0), (q, oracle.q_multiplier(SCALE))):
        codes, scales = oracle.quant_qk(x, mult)
        y = (x.float() * torch.tensor(mult, dtype=torch.float32)).permute(0, 2, 1, 3)
        y = torch.nn.functional.pad(y, (0, 0, 0, 256 - 200))
        blocks = y.reshape(1, 2, 8, 32, 128)
        amax = blocks.abs().amax(dim=(-1, -2))
        s = amax / torch.tensor(127.0)
        ref = torch.where(s[..., None, None] > 0, torch.round(blocks / s[..., None, None]), torch.zeros(()))
        ref = ref.clamp(-127, 127).to(torch.int8).reshape(1, 2, 256, 128)
        assert np.array_equal(scales, s.numpy())
        assert np.array_equal(codes, ref.numpy())


def test_quant_v_transpose_and_scales():
    B, S, H, D = 1, 300, 2, 128
    _, _, v = rand_qkv(B, S, H, D, seed=18)
    codes, scales = oracle.quant_v(v)
    assert codes.shape == (1, 2, 128, 512) and scales.shape == (1, 2, 128)
    vf = v.float().numpy()
    amax = np.abs(vf).max(axis=1)  # [B,H,D]
    assert np.array_equal(scales, (amax / np.float32(448.0)).astype(np.float32))
    ref = (torch.from_numpy(vf / scales[:, None, :, :]).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert np.array_equal(codes[:, :, :, :S], np.transpose(ref, (0, 2, 3, 1)))
    assert not codes[:, :, :, S:].any()
    # the absmax token of every channel reaches the largest code
    top = np.abs(vf).argmax(axis=1)
    for h in range(H):
        for ch in range(D):
            assert codes[0, h, ch, top[0, h, ch]] & 0x7F == 0x7E


# --------------------------------------------------------------------------
# cost model against the table the handbook page prints
# --------------------------------------------------------------------------

def test_cost_model_reproduces_printed_table():
    import json
    import os
    from image_dit_amd import cost
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attn_cost_table.json")))
    GiB = 1024.0 ** 3
    for row in g["attn_bytes_rows"]:
        n, h = row["tokens"], row["heads"]
        assert round(cost.score_matrix_bytes(1, h, n) / GiB, 1) == row["scores_gib"]
        assert round(cost.naive_attn_bytes(1, h, n, 128) / GiB, 1) == row["naive_gib"]
        assert round(cost.attn_bytes_bf16(1, h, n, 128) / GiB, 2) == row["flash_gib"]
    fr = g["flash_block_profile_row"]
    heads = fr["d_model"] // 128
    flops = cost.attn_flops(1, heads, fr["n"], 128)
    byts = cost.attn_bytes_bf16(1, heads, fr["n"], 128)
    assert round(flops / 1e9, 1) == fr["gflop"]
    assert round(byts / 2 ** 20) == fr["traffic_mib"]
    assert round(flops / byts) == fr["intensity"]
    assert round(max(flops / fr["peak_flops"], byts / fr["bandwidth"]) * 1e6) == fr["time_us"]


# --------------------------------------------------------------------------
# Q/K row transform: RMSNorm + rotate-half RoPE, BF16 rounding
# ("gfx1201_sage_prepare / gfx1201_sage_attention", first commit and
# "Technical Details": rounded like the eager PyTorch BF16 sequence)
# --------------------------------------------------------------------------

def torch_eager_norm_rope(x, w, eps, cos, sin, rope_dim):
    """The eager PyTorch BF16 sequence, op by op (each op rounds to BF16)."""
    y = x
    if w is not None:
        xf = y.float()
        y = (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps)).to(torch.bfloat16) * w
    if rope_dim:
        S = x.shape[1]
        half = rope_dim // 2
        yr, yp = y[..., :rope_dim], y[..., rope_dim:]
        rot = torch.cat((-yr[..., half:], yr[..., :half]), dim=-1)
        c = cos[:S].view(1, S, 1, rope_dim)
        s = sin[:S].view(1, S, 1, rope_dim)
        y = torch.cat((yr * c + rot * s, yp), dim=-1)
    return y


def rope_tables(S, rope_dim, base=10000.0):
    """BF16 cos/sin tables [S, rope_dim] of the rotate-half form (halves repeat)."""
    half = rope_dim // 2
    inv = 1.0 / base ** (torch.arange(half, dtype=torch.float64) / half)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * inv[None, :]
    ang = torch.cat((ang, ang), dim=-1)
    return torch.cos(ang).to(torch.bfloat16), torch.sin(ang).to(torch.bfloat16)


def as_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def test_f32_to_bf16_rounds_to_nearest_even():
    g = torch.Generator().manual_seed(11)
    vals = torch.randn(3000, generator=g) * torch.exp2(torch.randint(-40, 40, (3000,), generator=g).float())
    # exact midpoints between BF16 neighbours, with even and odd upper halves
    hi = torch.randint(0x0080, 0x7F00, (2000,), generator=g, dtype=torch.int32)
    mids = ((hi << 16) | 0x8000).view(torch.float32)
    for x in torch.cat((vals, mids, -mids)).tolist():
        ref = int(torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        assert oracle.f32_to_bf16(x) == ref, x


@pytest.mark.parametrize("rope_dim", [0, 32, 64, 96, 128])
@pytest.mark.parametrize("norm", [False, True])
def test_norm_rope_equals_torch_eager_on_exact_sums(rope_dim, norm):
    # inputs k/16 with |k| < 128: every square is a multiple of 2^-8 below 64, so
    # the fp32 sum of squares is exact in any order and torch must agree bitwise
    B, S, H, D = 2, 40, 3, 128
    g = torch.Generator().manual_seed(100 + rope_dim + norm)
    x = (torch.randint(-127, 128, (B, S, H, D), generator=g).float() / 16).to(torch.bfloat16)
    w = (1 + 0.25 * torch.randn(D, generator=g)).to(torch.bfloat16) if norm else None
    cos, sin = rope_tables(S + 5, rope_dim) if rope_dim else (None, None)
    ref = torch_eager_norm_rope(x, w, 1e-6, cos, sin, rope_dim)
    got = as_bf16(oracle.qk_norm_rope(x, w, 1e-6, cos, sin, rope_dim))
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("rope_dim", [32, 96, 128])
def test_norm_rope_close_to_torch_eager_on_randn(rope_dim):
    # random rows: only the (unspecified) order of torch's fp32 sum of squares can
    # differ, which moves a BF16 result by at most one unit in the last place
    B, S, H, D = 1, 64, 4, 128
    g = torch.Generator().manual_seed(7 + rope_dim)
    x = (3 * torch.randn((B, S, H, D), generator=g)).to(torch.bfloat16)
    w = (1 + 0.25 * torch.randn(D, generator=g)).to(torch.bfloat16)
    cos, sin = rope_tables(S, rope_dim)
    ref = torch_eager_norm_rope(x, w, 1e-6, cos, sin, rope_dim)
    got = as_bf16(oracle.qk_norm_rope(x, w, 1e-6, cos, sin, rope_dim))
    same = (got.view(torch.int16) == ref.view(torch.int16)).float().mean().item()
    assert same >= 0.99, same
    ulp = torch.abs(got.float() - ref.float()) / torch.exp2(torch.floor(torch.log2(ref.float().abs().clamp_min(1e-30))) - 7)
    assert ulp.max().item() <= 2.0


def test_rmsnorm_closed_forms():
    D = 128
    # constant row a: mean square a^2, so x * rsqrt(a^2) = sign(a) exactly (eps = 0)
    for a in (0.5, -3.0, 1.0, 96.0):
        x = torch.full((1, 1, 1, D), a).to(torch.bfloat16)
        got = as_bf16(oracle.qk_norm_rope(x, torch.ones(D, dtype=torch.bfloat16), 0.0))
        assert torch.equal(got.float(), torch.full((1, 1, 1, D), math.copysign(1.0, a)))
    # one nonzero channel a: x * r = sign(a) * sqrt(128), rounded to BF16 = 11.3125
    x = torch.zeros((1, 1, 1, D))
    x[..., 5] = 4.0
    got = as_bf16(oracle.qk_norm_rope(x.to(torch.bfloat16), torch.ones(D, dtype=torch.bfloat16), 0.0)).float()
    assert got[0, 0, 0, 5].item() == 11.3125 and float(got.abs().sum()) == 11.3125
    # the weight multiplies channel by channel
    w = torch.arange(1, D + 1, dtype=torch.float32).to(torch.bfloat16)
    x = torch.full((1, 1, 1, D), 2.0).to(torch.bfloat16)
    got = as_bf16(oracle.qk_norm_rope(x, w, 0.0)).float()
    assert torch.equal(got.flatten(), w.float())


@pytest.mark.parametrize("rope_dim", [32, 64, 96, 128])
def test_rope_special_tables(rope_dim):
    B, S, H, D = 1, 9, 2, 128
    g = torch.Generator().manual_seed(rope_dim)
    x = torch.randn((B, S, H, D), generator=g).to(torch.bfloat16)
    one = torch.ones((S, rope_dim), dtype=torch.bfloat16)
    zero = torch.zeros((S, rope_dim), dtype=torch.bfloat16)
    # angle 0: identity
    assert torch.equal(as_bf16(oracle.qk_norm_rope(x, None, 0.0, one, zero, rope_dim)), x)
    # angle pi/2: exactly rotate_half on the rotated channels, the rest untouched
    got = as_bf16(oracle.qk_norm_rope(x, None, 0.0, zero, one, rope_dim))
    half = rope_dim // 2
    exp = x.clone()
    exp[..., :half] = -x[..., half:rope_dim]
    exp[..., half:rope_dim] = x[..., :half]
    assert torch.equal(got, exp)


def test_rope_matches_the_rotation_in_fp64():
    # pins the pairing of channel c with c + rope_dim/2, the sign of the rotated
    # half and the position index of the table row
    B, S, H, D, rd = 1, 50, 2, 128, 64
    g = torch.Generator().manual_seed(5)
    x = torch.randn((B, S, H, D), generator=g).to(torch.bfloat16)
    cos, sin = rope_tables(S, rd)
    got = as_bf16(oracle.qk_norm_rope(x, None, 0.0, cos, sin, rd)).double()
    xd, cd, sd = x.double(), cos.double()[None, :, None, :], sin.double()[None, :, None, :]
    half = rd // 2
    x1, x2 = xd[..., :half], xd[..., half:rd]
    exp = torch.cat((x1 * cd[..., :half] - x2 * sd[..., :half], x2 * cd[..., half:] + x1 * sd[..., half:]), -1)
    err = (got[..., :rd] - exp).abs().max().item()
    assert err <= 3 * 2.0 ** -8 * xd.abs().max().item(), err
    assert torch.equal(got[..., rd:], xd[..., rd:])


# --------------------------------------------------------------------------
# K smoothing ("Kernel acceleration: attention, compilation and fusion",
# section "SageAttention: quantizing attention too")
# --------------------------------------------------------------------------

def test_channel_mean_is_the_rounded_exact_mean():
    # fp32(fp64(exact sum) / S): math.fsum gives the exactly rounded sum
    B, S, H, D = 2, 777, 3, 128
    _, k, _ = synth.make_qkv(B, S, H, D, seed=21, k_bias_std=2.0)
    got = oracle.channel_mean(k)
    kd = k.double().numpy()
    for b, h, d in [(0, 0, 0), (1, 2, 127), (0, 1, 64), (1, 0, 5)]:
        exact = math.fsum(kd[b, :, h, d].tolist())
        assert got[b, h, d] == np.float32(exact / S)
    ref = np.float32(kd.sum(axis=1) / S)  # [B, H, D]; the fp64 sum is exact here, any order agrees
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_smoothing_constant_keys_gives_zero_codes():
    # every key equal to u: the mean is u exactly and the smoothed K is 0
    B, S, H, D = 1, 96, 2, 128
    u = torch.randn((1, 1, H, D), generator=torch.Generator().manual_seed(3))
    k = bf16(u.expand(B, S, H, D).contiguous())
    mean = oracle.channel_mean(k)
    assert np.array_equal(mean, k[0, 0].float().numpy()[None])
    codes, scales = oracle.quant_qk(k, 1.0, mean)
    assert not codes.any() and not scales.any()


def test_smoothed_quant_matches_torch_vectorized():
    B, S, H, D = 1, 100, 2, 128
    _, k, _ = synth.make_qkv(B, S, H, D, seed=22, k_bias_std=2.0)
    mean = oracle.channel_mean(k)
    codes, scales = oracle.quant_qk(k, 1.0, mean)
    y = k.float().permute(0, 2, 1, 3) - torch.from_numpy(mean)[:, :, None, :]  # [B, H, S, D]
    Sp = oracle.sage_padded_len(S)
    y = torch.nn.functional.pad(y, (0, 0, 0, Sp - S)).reshape(B, H, Sp // 32, 32 * D)
    amax = y.abs().amax(-1)
    s = amax / 127.0
    ref = torch.where(s[..., None] > 0, torch.round(y / s[..., None]), torch.zeros(()))
    ref = ref.clamp(-127, 127).to(torch.int8).reshape(B, H, Sp, D)
    assert torch.equal(torch.from_numpy(scales), s)
    assert torch.equal(torch.from_numpy(codes), ref)
    # smoothing shrinks the block scales of a K with per-channel bias
    _, plain = oracle.quant_qk(k, 1.0)
    assert float(scales[:, :, : S // 32].mean()) < 0.7 * float(plain[:, :, : S // 32].mean())


# --------------------------------------------------------------------------
# exact attention with S_q != S_kv, grouped heads and a key window
# ("RDNAttention" README, "Features")
# --------------------------------------------------------------------------

def sdpa_masked_f64(q, k, v, scale, wl, wr):
    """torch SDPA in float64 with an explicit boolean mask and K/V heads repeated."""
    B, S_q, H, D = q.shape
    S_kv, H_kv = k.shape[1], k.shape[2]
    G = H // H_kv
    qd = q.double().permute(0, 2, 1, 3)
    kd = k.double().permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vd = v.double().permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    i = torch.arange(S_q)[:, None] + (S_kv - S_q)
    j = torch.arange(S_kv)[None, :]
    mask = torch.ones((S_q, S_kv), dtype=torch.bool)
    if wl >= 0:
        mask &= j >= i - wl
    if wr >= 0:
        mask &= j <= i + wr
    out = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask, scale=scale)
    return out.permute(0, 2, 1, 3).numpy(), mask.any(dim=1).numpy()


@pytest.mark.parametrize("S_q,S_kv,H,H_kv,wl,wr", [
    (50, 50, 4, 4, -1, -1), (37, 90, 4, 2, -1, -1), (90, 37, 6, 1, -1, -1),   # cross, GQA, MQA
    (70, 70, 2, 2, -1, 0), (40, 100, 2, 1, -1, 0), (100, 40, 2, 2, -1, 0),   # causal, aligned at the end
    (80, 80, 2, 2, 9, 0), (80, 80, 4, 2, 7, 7), (60, 90, 2, 2, 0, 12), (1, 77, 3, 3, -1, 0)])
def test_attn_rows_ex_matches_sdpa_with_mask(S_q, S_kv, H, H_kv, wl, wr):
    g = torch.Generator().manual_seed(S_q * 7 + S_kv + wl + 3 * wr)
    B = 2
    q = torch.randn((B, S_q, H, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, S_kv, H_kv, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, S_kv, H_kv, 128), generator=g).to(torch.bfloat16)
    got = oracle.attn_rows_ex(q, k, v, SCALE, (wl, wr))
    ref, seen = sdpa_masked_f64(q, k, v, SCALE, wl, wr)
    assert np.max(np.abs(got[:, seen] - ref[:, seen])) < 1e-12
    assert not got[:, ~seen].any()  # rows that see no key are zero


def test_attn_rows_ex_closed_forms():
    B, S, H = 1, 64, 2
    q, k, v = rand_qkv(B, S, H, seed=31)
    # a window of one key returns that key's value
    got = oracle.attn_rows_ex(q, k, v, SCALE, (0, 0))
    assert np.array_equal(got, v.double().numpy())
    # causal: the first query sees only the first key
    got = oracle.attn_rows_ex(q, k, v, SCALE, (-1, 0))
    assert np.array_equal(got[:, 0], v[:, 0].double().numpy())
    # full window equals plain self-attention
    assert np.max(np.abs(oracle.attn_rows_ex(q, k, v, SCALE) - oracle.attn_rows(q, k, v, SCALE))) < 1e-12
    # a decode step (one query) under the causal mask sees every key
    qd = q[:, -1:].contiguous()
    a = oracle.attn_rows_ex(qd, k, v, SCALE, (-1, 0))
    full = oracle.attn_rows(q, k, v, SCALE)[:, -1:]
    assert np.max(np.abs(a - full)) < 1e-12
    # single key/value head shared by every query head
    k1, v1 = k[:, :, :1].contiguous(), v[:, :, :1].contiguous()
    got = oracle.attn_rows_ex(q, k1, v1, SCALE)
    for h in range(H):
        ref = oracle.attn_rows(q[:, :, h:h + 1].contiguous(), k1, v1, SCALE)
        assert np.max(np.abs(got[:, :, h:h + 1] - ref)) < 1e-12


def test_thread_count_of_one_call_does_not_stick():
    # a one-thread call must leave later calls on the default team size
    before = oracle.num_threads()
    q, k, v = rand_qkv(1, 64, 2, seed=41)
    rows = np.array([[0, 0, 5], [0, 1, 63]], dtype=np.int64)
    a = oracle.attn_rows(q, k, v, SCALE, rows=rows, nthreads=1)
    b = oracle.attn_rows_ex(q, k, v, SCALE, (-1, 0), rows=rows, nthreads=1)
    assert oracle.num_threads() == before
    assert np.array_equal(a, oracle.attn_rows(q, k, v, SCALE, rows=rows))
    assert np.array_equal(b, oracle.attn_rows_ex(q, k, v, SCALE, (-1, 0), rows=rows))


# --------------------------------------------------------------------------
# attention of the quantized operands
# --------------------------------------------------------------------------

def exact_qk(g, B, S, H, D=128):
    """Q or K values the quantizer represents exactly: each 32-row block holds integers c in
    [-127, 127] (one of them +-127) times its own power of two."""
    nblk = -(-S // 32)
    c = g.integers(-127, 128, size=(B, S, H, D))
    e = g.integers(-7, -4, size=(B, nblk, H))          # 2^-7 .. 2^-5 per block
    for b in range(B):
        for blk in range(nblk):
            for h in range(H):
                c[b, 32 * blk + g.integers(0, min(32, S - 32 * blk)), h, g.integers(0, D)] = \
                    127 * (1 if g.random() < 0.5 else -1)
    return bf16(c * np.exp2(np.repeat(e, 32, axis=1)[:, :S, :, None]))


def exact_v(g, B, S, H, D=128):
    """V values the quantizer represents exactly: each channel holds E4M3 values (one of them
    448) times its own power of two."""
    mags = np.array([oracle.e4m3_decode(cd) for cd in range(127)])
    vm = mags[g.integers(0, 127, size=(B, S, H, D))] * np.where(g.random((B, S, H, D)) < 0.5, 1, -1)
    for b in range(B):
        for h in range(H):
            for d in range(D):
                vm[b, g.integers(0, S), h, d] = 448.0
    ev = g.integers(-10, -5, size=(B, 1, H, D))             # 2^-10 .. 2^-6 per channel
    return bf16(vm * np.exp2(ev))


def exactly_quantizable(B, S, H, seed, D=128):
    g = np.random.default_rng(seed)
    return exact_qk(g, B, S, H, D), exact_qk(g, B, S, H, D), exact_v(g, B, S, H, D)


@pytest.mark.parametrize("B,S,H", [(1, 64, 1), (2, 100, 3)])
def test_sage_attn_rows_is_exact_attention_on_exact_codes(B, S, H):
    # On inputs the quantizer represents exactly, attention of the quantized operands is exact
    # attention up to the fp32 rounding of Q's multiplier (relative 2^-23 per score); a wrong
    # scale block, V transpose, V channel scale or base of the softmax fails by far more.
    q, k, v = exactly_quantizable(B, S, H, seed=B * 1000 + S)
    prep = oracle.sage_prepare(q, k, v, SCALE)
    qc, qs, kc, ks, vc, vs = prep
    # the premise: codes times scales give back the inputs (Q times its multiplier)
    mult = oracle.q_multiplier(SCALE)
    kd = kc[:, :, :S].astype(np.float64) * np.repeat(ks, 32, axis=2)[:, :, :S, None]
    assert np.array_equal(kd, f64(k).transpose(0, 2, 1, 3))
    qd = qc[:, :, :S].astype(np.float64) * np.repeat(qs, 32, axis=2)[:, :, :S, None]
    np.testing.assert_allclose(qd, f64(q).transpose(0, 2, 1, 3) * mult, rtol=2e-7, atol=0)
    dec = np.array([oracle.e4m3_decode(cd) for cd in range(256)])
    vd = dec[vc[:, :, :, :S]] * vs[:, :, :, None]
    assert np.array_equal(vd, f64(v).transpose(0, 2, 3, 1))
    rows = np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(S)])
    got = oracle.sage_attn_rows(prep, S, rows)
    ref = oracle.attn_rows(q, k, v, SCALE, rows=rows)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5 * np.abs(ref).max())


def test_sage_attn_rows_single_key_and_equal_scores():
    # S = 1: the output is the key's decoded V row.  Q = 0: every weight equal, so the output is
    # the mean of the decoded V rows.
    q, k, v = rand_qkv(1, 40, 2, seed=5)
    for S in (1, 40):
        qq = torch.zeros_like(q[:, :S]) if S > 1 else q[:, :S]
        prep = oracle.sage_prepare(qq, k[:, :S], v[:, :S], SCALE)
        qc, qs, kc, ks, vc, vs = prep
        dec = np.array([oracle.e4m3_decode(cd) for cd in range(256)])
        vd = dec[vc[:, :, :, :S]] * vs[:, :, :, None]          # [B, H, D, S]
        rows = np.array([(0, h, i) for h in range(2) for i in range(S)])
        got = oracle.sage_attn_rows(prep, S, rows)
        want = np.stack([vd[0, r[1]].mean(axis=1) for r in rows])
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)


def test_sage_attn_rows_error_is_the_quantizers():
    # On randn inputs the quantized operands' attention stays within the gates the kernels are
    # held to against exact attention (cosine >= 0.998, relative L2 <= 0.05), and is not exact
    # (INT8 Q/K and FP8 V do change the result).
    q, k, v = rand_qkv(1, 256, 2, seed=9)
    rows = np.array([(0, h, i) for h in range(2) for i in range(0, 256, 3)])
    got = oracle.sage_attn_rows(oracle.sage_prepare(q, k, v, SCALE), 256, rows)
    ref = oracle.attn_rows(q, k, v, SCALE, rows=rows)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    cos = (got * ref).sum() / np.linalg.norm(got) / np.linalg.norm(ref)
    assert 1e-3 < rel <= 0.05 and cos >= 0.998, (rel, cos)


@pytest.mark.parametrize("B,S_q,S_kv,H,H_kv,window", [
    (2, 70, 300, 4, 2, (-1, -1)),    # cross-attention, grouped heads, S_kv padded to 512
    (1, 150, 70, 3, 1, (-1, 0)),     # causal with S_q > S_kv: the first 80 rows see no key
    (1, 100, 100, 2, 2, (20, 5)),    # two-sided window
    (1, 1, 90, 4, 4, (-1, 0)),       # a decode step sees every key
])
def test_sage_attn_rows_ex_is_exact_windowed_attention_on_exact_codes(B, S_q, S_kv, H, H_kv, window):
    # as above, with the key/value head of each query head, the window and empty rows
    g = np.random.default_rng(S_q * 7 + S_kv)
    q, k, v = exact_qk(g, B, S_q, H), exact_qk(g, B, S_kv, H_kv), exact_v(g, B, S_kv, H_kv)
    prep = oracle.sage_prepare_ex(q, k, v, SCALE)
    rows = np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(S_q)])
    got = oracle.sage_attn_rows_ex(prep, S_q, S_kv, window, rows)
    ref = oracle.attn_rows_ex(q, k, v, SCALE, window, rows=rows)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5 * np.abs(ref).max())
    if window == (-1, 0) and S_q > S_kv:
        assert not got[rows[:, 2] < S_q - S_kv].any()

