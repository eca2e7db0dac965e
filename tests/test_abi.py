"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments before anything is enqueued
(argument checks touch no HIP API, so they run on any host)."""
import ctypes
import os
import re
import subprocess

import pytest

import image_dit_amd as ia

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ditattn.h")

EINVAL, EUNSUPPORTED, EALIGN, EOVERFLOW = -1, -2, -3, -4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ia.LIB_PATH):
        from image_dit_amd import build
        build.build(force=False)
    return ia.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_fwd_bf16", "sage_prepare", "sage_attn_fwd", "ditattn_sage_padded_len",
              "ditattn_status_string", "ditattn_abi_version", "ditattn_check_shape"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ia.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_library_links_only_the_hip_runtime():
    out = subprocess.run(["ldd", ia.LIB_PATH], capture_output=True, text=True, check=True).stdout
    libs = {line.split()[0] for line in out.splitlines() if "=>" in line}
    allowed = re.compile(r"^(libamdhip64|libstdc\+\+|libm|libgcc_s|libc|librocprofiler-register|"
                         r"libhsa-runtime64|libelf|libdrm|libdrm_amdgpu|libnuma|libz)\.so")
    bad = [x for x in libs if not allowed.match(x)]
    assert not bad, bad  # no BLAS, DNN or attention library


def test_abi_version_and_padded_len(lib):
    assert lib.ditattn_abi_version() == 1
    assert [lib.ditattn_sage_padded_len(s) for s in (1, 256, 257, 4608, 76112)] == [256, 256, 512, 4608, 76288]
    assert lib.ditattn_sage_padded_len(0) == -1
    assert lib.ditattn_sage_padded_len(2**31 - 1) == -1
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(lib.ditattn_status_string(st), bytes)


GOOD = 0x1000  # an aligned fake device address; argument errors return before any use


def bf16_call(lib, q=GOOD, k=GOOD * 2 ** 20, v=GOOD * 2 ** 21, o=GOOD * 2 ** 22, B=1, S=64, H=2, D=128, scale=0.088):
    return lib.attn_fwd_bf16(ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), ctypes.c_void_p(o),
                             B, S, H, D, ctypes.c_float(scale), None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), EINVAL), (dict(S=0), EINVAL), (dict(H=-1), EINVAL),
    (dict(scale=0.0), EINVAL), (dict(scale=-1.0), EINVAL), (dict(scale=float("nan")), EINVAL),
    (dict(scale=float("inf")), EINVAL), (dict(q=0), EINVAL), (dict(o=0), EINVAL),
    (dict(D=64), EUNSUPPORTED), (dict(D=256), EUNSUPPORTED),
    (dict(k=GOOD * 2 ** 20 + 8), EALIGN), (dict(o=GOOD * 2 ** 22 + 2), EALIGN),
    (dict(o=GOOD), EINVAL),  # output aliases q
    (dict(o=GOOD + 64 * 2 * 128 * 2 - 16), EINVAL),  # partial overlap with q
    (dict(B=2 ** 16, H=2 ** 16), EOVERFLOW), (dict(S=2 ** 31 - 100), EOVERFLOW),
])
def test_attn_fwd_bf16_rejects(lib, kw, status):
    assert bf16_call(lib, **kw) == status


def prep_call(lib, override=None, B=1, S=100, H=2, D=128, scale=0.088):
    ptrs = [GOOD * 2 ** (20 + i) for i in range(9)]
    for i, val in (override or {}).items():
        ptrs[i] = val
    return lib.sage_prepare(*[ctypes.c_void_p(p) for p in ptrs], B, S, H, D, ctypes.c_float(scale), None)


def test_sage_prepare_rejects(lib):
    assert prep_call(lib, B=0) == EINVAL
    assert prep_call(lib, D=96) == EUNSUPPORTED
    assert prep_call(lib, scale=float("nan")) == EINVAL
    for i in range(9):
        assert prep_call(lib, {i: 0}) == EINVAL
        assert prep_call(lib, {i: GOOD * 2 ** (20 + i) + 4}) == EALIGN
    assert prep_call(lib, {3: GOOD * 2 ** 20}) == EINVAL  # q_i8 over q
    assert prep_call(lib, {5: GOOD * 2 ** 23}) == EINVAL  # k_i8 over q_i8


def attn_call(lib, override=None, B=1, S=100, H=2, D=128, scale=0.088):
    ptrs = [GOOD * 2 ** (20 + i) for i in range(7)]
    for i, val in (override or {}).items():
        ptrs[i] = val
    return lib.sage_attn_fwd(*[ctypes.c_void_p(p) for p in ptrs], B, S, H, D, ctypes.c_float(scale), None)


def test_sage_attn_fwd_rejects(lib):
    assert attn_call(lib, S=0) == EINVAL
    assert attn_call(lib, D=127) == EUNSUPPORTED
    assert attn_call(lib, scale=0.0) == EINVAL
    for i in range(7):
        assert attn_call(lib, {i: 0}) == EINVAL
        assert attn_call(lib, {i: GOOD * 2 ** (20 + i) + 8}) == EALIGN
    assert attn_call(lib, {6: GOOD * 2 ** 20}) == EINVAL  # o over q_i8


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("image_dit_amd")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="not found"):
            mod.load(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


# ---------------------------------------------------------------- size limits
# Every accepted shape must be one the kernels index without 32-bit wrap-around:
# the BF16 kernel forms K/V row offsets r * H * 256 (r < 64) in 32 bits, the Sage
# kernel forms V^T row offsets c * S_pad (c < 128) in 32 bits, and tile/grid
# indices are int (B * H * S_pad <= INT32_MAX).  Only the host checks run here.
ENTRY_BF16, ENTRY_PREP, ENTRY_SAGE = 0, 1, 2
MAX_HEADS, MAX_SEQ_SAGE = 65536, 1 << 25


def check_shape(lib, entry, B, S, H, D=128, scale=0.088):
    lib.ditattn_check_shape.argtypes = [ctypes.c_int] * 5 + [ctypes.c_float]
    return lib.ditattn_check_shape(entry, B, S, H, D, scale)


def test_limits_are_in_kernel_index_range():
    # the arithmetic the bounds rest on
    assert 63 * MAX_HEADS * 256 + 16 * 15 < 2 ** 32
    assert 63 * (MAX_HEADS + 1) * 256 < 2 ** 32  # H itself is bounded more tightly than needed
    assert 127 * MAX_SEQ_SAGE + 16 * 3 < 2 ** 32 and MAX_SEQ_SAGE % 256 == 0
    assert 127 * (MAX_SEQ_SAGE + 256) >= 2 ** 32 - 2 ** 26  # next padded length is close to the wrap


@pytest.mark.parametrize("entry", [ENTRY_BF16, ENTRY_PREP, ENTRY_SAGE])
def test_heads_limit(lib, entry):
    assert check_shape(lib, entry, 1, 256, MAX_HEADS) == 0
    assert check_shape(lib, entry, 1, 256, MAX_HEADS + 1) == EOVERFLOW


@pytest.mark.parametrize("entry", [ENTRY_BF16, ENTRY_PREP, ENTRY_SAGE])
def test_total_rows_limit(lib, entry):
    # B * H * S_pad <= INT32_MAX: 8192 * 261888 fits, 8192 * 262144 = 2^31 does not
    assert check_shape(lib, entry, 1, 261888, 8192) == 0
    assert check_shape(lib, entry, 1, 261889, 8192) == EOVERFLOW
    assert check_shape(lib, entry, 2, 130816, 8192) == 0  # 2 * 8192 * 130816 < 2^31
    assert check_shape(lib, entry, 2, 130817, 8192) == EOVERFLOW  # S_pad 131072


def test_sage_sequence_limit(lib):
    assert check_shape(lib, ENTRY_SAGE, 1, MAX_SEQ_SAGE, 1) == 0
    assert check_shape(lib, ENTRY_SAGE, 1, MAX_SEQ_SAGE + 1, 1) == EOVERFLOW
    # the prepare stage and the BF16 path index nothing in units of S_pad * 128
    assert check_shape(lib, ENTRY_PREP, 1, MAX_SEQ_SAGE + 1, 1) == 0
    assert check_shape(lib, ENTRY_BF16, 1, MAX_SEQ_SAGE + 1, 1) == 0
    # and the entry point itself rejects before looking at pointers
    assert attn_call(lib, S=MAX_SEQ_SAGE + 1) == EOVERFLOW
    assert bf16_call(lib, H=MAX_HEADS + 1) == EOVERFLOW
    assert prep_call(lib, H=MAX_HEADS + 1) == EOVERFLOW


def test_check_shape_matches_argument_rules(lib):
    assert check_shape(lib, ENTRY_BF16, 0, 64, 2) == EINVAL
    assert check_shape(lib, ENTRY_BF16, 1, 64, 2, D=64) == EUNSUPPORTED
    assert check_shape(lib, ENTRY_BF16, 1, 64, 2, scale=float("nan")) == EINVAL
    assert check_shape(lib, 7, 1, 64, 2) == EINVAL


# ---------------------------------------------------------------- binding output checks
def test_binding_rejects_wrong_outputs_before_any_call(monkeypatch):
    import torch
    mod = ia
    calls = []

    class FakeLib:
        def __getattr__(self, name):
            def f(*a):
                calls.append(name)
                return 0
            return f

        def ditattn_sage_padded_len(self, S):
            return (S + 255) // 256 * 256

    monkeypatch.setattr(mod, "load", lambda path=None: FakeLib())
    dev = torch.device("meta")
    q = torch.empty((1, 300, 2, 128), dtype=torch.bfloat16, device=dev)
    monkeypatch.setattr(mod, "_check_bshd", lambda name, t, dtype: None)
    monkeypatch.setattr(mod, "_stream_handle", lambda s: None)
    short = torch.empty((1, 299, 2, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="shape"):
        mod.attn_fwd_bf16(q, q, q, 0.088, out=short)
    wrong_dtype = torch.empty((1, 300, 2, 128), dtype=torch.float16, device=dev)
    with pytest.raises(ValueError, match="bfloat16"):
        mod.attn_fwd_bf16(q, q, q, 0.088, out=wrong_dtype)
    good = [torch.empty(shape, dtype=dt, device=dev) for _, shape, dt in mod._prepared_specs(1, 300, 2, 128)]
    for i in range(6):
        bad = list(good)
        bad[i] = torch.empty((1,), dtype=good[i].dtype, device=dev)
        with pytest.raises(ValueError):
            mod.sage_prepare(q, q, q, 0.088, out=tuple(bad))
        with pytest.raises(ValueError):
            mod.sage_attn_fwd(tuple(bad), 300, 2, 0.088)
    with pytest.raises(ValueError):
        mod.sage_prepare(q, q, q, 0.088, out=tuple(good[:5]))
    assert calls == []  # nothing reached the library
