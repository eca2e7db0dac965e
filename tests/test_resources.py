"""Resource audit of the gfx950 kernels, on the CPU: every kernel is compiled with the
library's own flags and the compiler's resource report is checked against the budgets the
kernels are designed for.  No GPU is needed (hipcc cross-compiles).

Budgets:
  * no kernel spills registers or uses scratch memory (a spill inside the key loop turns
    the attention kernels memory-bound);
  * the attention kernels run 8 waves per workgroup, two per SIMD (the ping-pong pairs
    waves w and w + 4 on one SIMD), so the compiler must report an occupancy of at least
    two waves per SIMD, i.e. at most 256 VGPRs + AGPRs per wave;
  * LDS per workgroup: BF16 four 16 KB K/V stages (64 KB), Sage three 16 KB K + V^T stages
    plus the k_scale pairs, one code-path flag per wave and the tile's v_scale (48 KB + 592 B); both far below the
    160 KB of a CU.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from image_dit_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "image_dit_amd", "csrc")

ATTENTION = {  # kernel name fragment -> max LDS bytes per workgroup
    "attn_fwd_bf16_kernel": 65536 + 64,
    "attn_fwd_bf16_split_kernel": 65536 + 64,
    "sage_attn_fwd_kernel": 3 * (8192 + 8192) + 64 + 32 + 512,
    "sage_attn_fwd_split_kernel": 3 * (8192 + 8192) + 64 + 32 + 512,
}


def _hipcc():
    try:
        return libbuild.hipcc()
    except RuntimeError:
        return None


def _report(src):
    """{kernel mangled name: {field: value}} from -Rpass-analysis=kernel-resource-usage."""
    flags = [f for f in libbuild.compile_flags() if f != "-fPIC"]
    cmd = [_hipcc()] + flags + ["--cuda-device-only", "-c", "-o", os.devnull,
                                "-Rpass-analysis=kernel-resource-usage", os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?):\s+(\S+)\s+\[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


@pytest.fixture(scope="module")
def reports():
    if _hipcc() is None:
        pytest.skip("hipcc for gfx950 not available")
    with ThreadPoolExecutor(max_workers=len(libbuild.SOURCES)) as ex:
        res = dict(zip(libbuild.SOURCES, ex.map(_report, libbuild.SOURCES)))
    return {name: fields for per_src in res.values() for name, fields in per_src.items()}


def test_every_kernel_is_reported(reports):
    names = " ".join(reports)
    for frag in list(ATTENTION) + ["quant_qk_kernel", "v_absmax_kernel", "v_quant_kernel",
                                   "k_colsum_kernel", "k_mean_kernel", "xform_kernel"]:
        assert frag in names, frag


# The split-tail kernels run the whole attention body once per work item in a loop, with the
# item's plan (tile, key range, merge range) live beside the body's own scalars: the compiler
# keeps some scalars in VGPR lanes (v_writelane / v_readlane, no scratch memory), outside the
# key loop.  The allowance caps that at its current size; every other kernel keeps everything
# in SGPRs.
SGPR_LANE_SPILL_ALLOWANCE = {"attn_fwd_bf16_split_kernel": 96, "sage_attn_fwd_split_kernel": 64}


def test_no_spills_no_scratch(reports):
    for name, f in reports.items():
        assert int(f["ScratchSize [bytes/lane]"]) == 0, (name, f)
        assert int(f["VGPRs Spill"]) == 0, (name, f)
        allow = max([v for k, v in SGPR_LANE_SPILL_ALLOWANCE.items() if k + "E" in name] + [0])
        assert int(f["SGPRs Spill"]) <= allow, (name, f)
        assert f.get("Dynamic Stack", "False") == "False", (name, f)


@pytest.mark.parametrize("frag", sorted(ATTENTION))
def test_attention_kernels_fit_two_waves_per_simd(reports, frag):
    hits = [(n, f) for n, f in reports.items() if frag + "E" in n or n.endswith(frag)]
    assert hits, frag
    for name, f in hits:
        assert int(f["Occupancy [waves/SIMD]"]) >= 2, (name, f)
        assert int(f["VGPRs"]) + int(f["AGPRs"]) <= 256, (name, f)
        assert int(f["LDS Size [bytes/block]"]) <= ATTENTION[frag], (name, f)
