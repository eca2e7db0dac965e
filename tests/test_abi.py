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
              "ditattn_status_string", "ditattn_abi_version", "ditattn_check_shape",
              "sage_prepare_ex", "qk_norm_rope_bf16", "ditattn_sage_workspace_size"):
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
    assert lib.ditattn_abi_version() == 2
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
    monkeypatch.setattr(mod, "_check_bshd", lambda name, t, dtype, device=None: None)
    monkeypatch.setattr(mod, "_stream_handle", lambda s, device=None: None)
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


def test_binding_rejects_workspaces_off_the_tensors_device(monkeypatch):
    """A workspace in host memory (or on another GPU) would hand the kernels a pointer they
    cannot use: the binding refuses it before any library call."""
    import torch
    mod = ia
    calls = []

    class FakeLib:
        def __getattr__(self, name):
            def f(*a):
                calls.append(name)
                return 0
            return f

        def ditattn_sage_padded_len(self, S):  # a size query, not a launch
            return (S + 255) // 256 * 256

    monkeypatch.setattr(mod, "load", lambda path=None: FakeLib())
    monkeypatch.setattr(mod, "_check_bshd", lambda name, t, dtype, device=None: None)
    monkeypatch.setattr(mod, "_stream_handle", lambda s, device=None: None)
    monkeypatch.setattr(mod, "bf16_workspace_size", lambda *a, **k: 4096)
    monkeypatch.setattr(mod, "sage_workspace_size", lambda *a, **k: 4096)
    dev = torch.device("meta")
    q = torch.empty((1, 300, 2, 128), dtype=torch.bfloat16, device=dev)
    host_ws = torch.zeros(8192, dtype=torch.uint8)  # host memory
    with pytest.raises(ValueError, match="workspace"):
        mod.attn_fwd_bf16_ws(q, q, q, 0.088, workspace=host_ws)
    with pytest.raises(ValueError, match="workspace"):
        mod.attn_fwd_bf16_ws(q, q, q, 0.088, workspace=torch.empty(100, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="workspace"):
        mod.sage_prepare_ex(q, q, q, 0.088, smooth_k=True, workspace=host_ws)
    assert calls == []


def test_check_helpers_reject_other_devices():
    import torch
    cpu = torch.zeros((2, 4), dtype=torch.uint8)
    with pytest.raises(ValueError):
        ia._check_workspace(cpu, 8, torch.device("cuda", 0))
    with pytest.raises(ValueError):
        ia._check_workspace(torch.zeros(4, dtype=torch.uint8), 8, torch.device("cpu"))  # too small
    assert ia._check_workspace(torch.zeros(16, dtype=torch.int32), 64, torch.device("cpu")) == 64

    with pytest.raises(TypeError):  # host tensors are never accepted as inputs
        ia._check_bshd("k", torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16), torch.bfloat16)


# ---------------------------------------------------------------- sage_prepare_ex / qk_norm_rope_bf16
def prep_ex_call(lib, override=None, B=1, S_q=100, S_kv=100, H=2, H_kv=2, D=128, scale=0.088,
                 norm=(None, None), eps=1e-6, rope=(None, None), rope_dim=0, k_mean=None, ws=None,
                 ws_bytes=0):
    ptrs = [GOOD * 2 ** (20 + i) for i in range(9)]
    for i, val in (override or {}).items():
        ptrs[i] = val
    vp = ctypes.c_void_p
    return lib.sage_prepare_ex(*[vp(p) for p in ptrs], B, S_q, S_kv, H, H_kv, D, ctypes.c_float(scale),
                               vp(norm[0]), vp(norm[1]), ctypes.c_float(eps), vp(rope[0]), vp(rope[1]),
                               rope_dim, vp(k_mean), vp(ws), ctypes.c_size_t(ws_bytes), None)


def test_sage_prepare_ex_rejects(lib):
    W = GOOD * 2 ** 40  # far from every other fake buffer
    assert prep_ex_call(lib, H=3, H_kv=2) == EINVAL  # H not a multiple of H_kv
    assert prep_ex_call(lib, S_kv=0) == EINVAL
    assert prep_ex_call(lib, eps=-1.0) == EINVAL
    assert prep_ex_call(lib, eps=float("inf")) == EINVAL
    for rd in (16, 48, 100, 256):
        assert prep_ex_call(lib, rope_dim=rd, rope=(W, W + 2 ** 24)) == EUNSUPPORTED
    assert prep_ex_call(lib, rope_dim=64, rope=(W, None)) == EINVAL
    assert prep_ex_call(lib, rope_dim=64, rope=(W + 4, W + 2 ** 24)) == EALIGN
    assert prep_ex_call(lib, norm=(W + 2, None)) == EALIGN
    # smoothing needs a workspace of the size the library states
    need = lib.ditattn_sage_workspace_size(1, 100, 2)
    assert need > 0
    assert prep_ex_call(lib, k_mean=W) == EINVAL
    assert prep_ex_call(lib, k_mean=W, ws=W + 2 ** 24, ws_bytes=need - 1) == EINVAL
    assert prep_ex_call(lib, k_mean=W + 8, ws=W + 2 ** 24, ws_bytes=need) == EALIGN
    # k_mean over the workspace, workspace over v
    assert prep_ex_call(lib, k_mean=W, ws=W, ws_bytes=need) == EINVAL
    assert prep_ex_call(lib, k_mean=W, ws=GOOD * 2 ** 22, ws_bytes=need) == EINVAL
    # RoPE tables under an output
    assert prep_ex_call(lib, rope_dim=32, rope=(GOOD * 2 ** 23, W)) == EINVAL
    assert prep_ex_call(lib, D=64) == EUNSUPPORTED


def test_workspace_size_is_positive_and_bounded(lib):
    lib.ditattn_sage_workspace_size.restype = ctypes.c_size_t
    for B, S, H in ((1, 256, 2), (1, 4608, 24), (1, 76112, 40), (4, 300, 5)):
        n = lib.ditattn_sage_workspace_size(B, S, H)
        assert 0 < n <= max(8 << 20, B * H * 1024 * 2)
    assert lib.ditattn_sage_workspace_size(0, 10, 1) == 0


def test_qk_norm_rope_rejects(lib):
    vp = ctypes.c_void_p
    W = GOOD * 2 ** 40

    def call(x=GOOD, out=GOOD * 2 ** 30, S=64, H=2, D=128, w=None, eps=1e-6, rope=(None, None), rd=0):
        return lib.qk_norm_rope_bf16(vp(x), vp(out), 1, S, H, D, vp(w), ctypes.c_float(eps), vp(rope[0]),
                                     vp(rope[1]), rd, None)
    assert call(x=0) == EINVAL
    assert call(D=256) == EUNSUPPORTED
    assert call(rd=40, rope=(W, W + 2 ** 24)) == EUNSUPPORTED
    assert call(eps=float("nan"), w=W) == EINVAL
    assert call(out=GOOD + 256) == EINVAL  # partial overlap; exact in-place is allowed
    assert call(w=GOOD * 2 ** 30 + 1024) == EINVAL  # weight inside the output


# ---------------------------------------------------------------- sage_prepare_ex_noalloc
ENOSPACE = -6


def test_static_scratch_size_matches_header():
    m = re.search(r"#define DITATTN_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == ia.STATIC_SCRATCH_BYTES


def test_noalloc_rejects_before_any_hip_call(lib):
    vp = ctypes.c_void_p
    W = GOOD * 2 ** 40

    def call(B=1, S=100, H=2, H_kv=2, k_mean=None):
        ptrs = [GOOD * 2 ** (20 + i) for i in range(9)]
        return lib.sage_prepare_ex_noalloc(*[vp(p) for p in ptrs], B, S, S, H, H_kv, 128,
                                           ctypes.c_float(0.088), None, None, ctypes.c_float(1e-6),
                                           None, None, 0, vp(k_mean), None)
    lib.ditattn_sage_workspace_size.restype = ctypes.c_size_t
    # smoothing whose partial sums exceed the static scratch: B*H rows of one token range each
    B, S, H = 128, 16, 256
    assert lib.ditattn_sage_workspace_size(B, S, H) > ia.STATIC_SCRATCH_BYTES
    assert call(B=B, S=S, H=H, H_kv=H, k_mean=W) == ENOSPACE
    assert "scratch" in lib.ditattn_status_string(ENOSPACE).decode()
    # argument errors come first, as in sage_prepare_ex
    assert call(H=3, H_kv=2, k_mean=W) == EINVAL
    assert call(H=3, H_kv=2) == EINVAL


# ---------------------------------------------------------------- sage_attn_fwd_ws
def test_sage_ws_rejects_before_any_hip_call(lib):
    vp = ctypes.c_void_p
    ptrs = [GOOD * 2 ** (20 + i) for i in range(7)]  # q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, o

    def call(B=1, S=64, H=2, D=128, wl=-1, wr=-1, o=None):
        p = list(ptrs)
        if o is not None:
            p[6] = o
        return lib.sage_attn_fwd_ws(*[vp(x) for x in p], B, S, S, H, H, D, ctypes.c_float(0.088), wl, wr,
                                    None, 0, None)
    assert call(D=64) == EUNSUPPORTED
    assert call(wl=-2) == EINVAL
    assert call(o=ptrs[6] + 2) == EALIGN
    assert call(o=ptrs[0]) == EINVAL  # output over the Q codes
    assert call(H=MAX_HEADS + 1) == EOVERFLOW
    # without a GPU the plan is "no split": the size is 0, equal to the BF16 path's
    for args in ((1, 4608, 4608, 24, 24, -1, -1), (1, 16896, 16896, 24, 24, -1, -1), (1, 0, 64, 2, 2, -1, -1)):
        assert lib.ditattn_sage_attn_workspace_size(*args) == lib.ditattn_bf16_workspace_size(*args)


def test_binding_sage_ws_rejects_host_workspace(monkeypatch):
    import torch
    mod = ia
    calls = []

    class FakeLib:
        def __getattr__(self, name):
            def f(*a):
                calls.append(name)
                return 0
            return f

        def ditattn_sage_padded_len(self, S):  # a size query, not a launch
            return (S + 255) // 256 * 256

    monkeypatch.setattr(mod, "load", lambda path=None: FakeLib())
    monkeypatch.setattr(mod, "_stream_handle", lambda s, device=None: None)
    monkeypatch.setattr(mod, "sage_attn_workspace_size", lambda *a, **k: 4096)
    monkeypatch.setattr(mod, "_on_device", lambda d: __import__("contextlib").nullcontext())

    class Cuda(torch.Tensor):  # meta tensors that report a GPU device
        @property
        def device(self):
            return torch.device("cuda", 0)
    specs = mod._prepared_specs(1, 300, 2, 128)
    prepared = tuple(torch.empty(shape, dtype=dt, device="meta").as_subclass(Cuda) for _, shape, dt in specs)
    out = torch.empty((1, 300, 2, 128), dtype=torch.bfloat16, device="meta").as_subclass(Cuda)
    with pytest.raises(ValueError, match="workspace"):
        mod.sage_attn_fwd_ws(prepared, 300, 300, 2, 2, 0.088, out=out,
                             workspace=torch.zeros(8192, dtype=torch.uint8))
    assert calls == []


# ---------------------------------------------------------------- attn_fwd_bf16_ws
def test_bf16_ws_rejects_before_any_hip_call(lib):
    vp = ctypes.c_void_p

    def call(B=1, S=64, H=2, D=128, wl=-1, wr=-1, o=GOOD * 2 ** 22):
        return lib.attn_fwd_bf16_ws(vp(GOOD), vp(GOOD * 2 ** 20), vp(GOOD * 2 ** 21), vp(o), B, S, S, H, H,
                                    D, ctypes.c_float(0.088), wl, wr, None, 0, None)
    assert call(D=64) == EUNSUPPORTED
    assert call(wl=-2) == EINVAL
    assert call(o=GOOD * 2 ** 22 + 2) == EALIGN
    assert call(o=GOOD) == EINVAL  # output over q
    assert call(H=MAX_HEADS + 1) == EOVERFLOW
    # without a GPU the plan is "no split", so the size is 0 and no workspace is needed
    assert lib.ditattn_bf16_workspace_size(1, 4608, 4608, 24, 24, -1, -1) == 0
    assert lib.ditattn_bf16_workspace_size(1, 0, 4608, 24, 24, -1, -1) == 0
