"""CPU checks of the C ABI: symbols, validation errors, workspace queries.

No compute call is made: every call here fails validation (or is a pure
host query) before the library touches the HIP runtime.
"""
import ctypes as C
import os
import re

import pytest

import orthogonal_fine_tuning_amd as oft
from orthogonal_fine_tuning_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "oft.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)


def test_status_strings_and_version():
    lib = _lib.load()
    assert lib.oft_abi_version() == 8
    for s in range(-6, 1):
        assert lib.oft_status_str(s)
    assert b"unknown" in lib.oft_status_str(-99)


def _desc(**kw):
    base = dict(M=64, K=256, segs=(128, 128, 128), b=16, x_dtype=oft.OFT_DT_F32, w_fmt=oft.OFT_W_INT4, g=32)
    base.update(kw)
    return oft.linear_desc(base["M"], base["K"], base["segs"], base["b"], base["x_dtype"], base["w_fmt"],
                           base["g"])


@pytest.mark.parametrize("kw,code", [
    (dict(b=8), _lib.OFT_EUNSUPPORTED),
    (dict(g=16), _lib.OFT_EUNSUPPORTED),
    (dict(K=96), _lib.OFT_ESHAPE),                 # K % 64
    (dict(K=320, g=128), _lib.OFT_ESHAPE),         # K % g
    (dict(segs=(120, 136, 128)), _lib.OFT_ESHAPE),  # segment % b
    (dict(segs=(16, 16, 16)), _lib.OFT_ESHAPE),    # N % 32
    (dict(x_dtype=7), _lib.OFT_EDTYPE),
    (dict(w_fmt=9), _lib.OFT_EDTYPE),
    (dict(M=-1), _lib.OFT_EINVAL),
    (dict(w_fmt=oft.OFT_W_FP4_E2M1), _lib.OFT_OK),  # FP4: the INT4 constraints
    (dict(w_fmt=oft.OFT_W_FP4_E2M1, g=16), _lib.OFT_EUNSUPPORTED),
    (dict(w_fmt=oft.OFT_W_FP4_E2M1, K=320, g=128), _lib.OFT_ESHAPE),
])
def test_linear_validation(kw, code):
    d = _desc(**kw)
    n = C.c_size_t(0)
    assert _lib.load().oft_linear_workspace_bytes(C.byref(d), 1, C.byref(n)) == code


@pytest.mark.parametrize("kw,code", [
    (dict(M=1 << 22), _lib.OFT_OK),                       # 32768 token tiles of 128 along grid y
    (dict(M=(1 << 22) + 1), _lib.OFT_EUNSUPPORTED),
    (dict(M=64, K=1984, segs=(1 << 20,), b=32), _lib.OFT_OK),  # N K = 2^31 - 2^26
    (dict(M=64, K=2048, segs=(1 << 20,), b=32), _lib.OFT_EUNSUPPORTED),  # N K = 2^31: 32-bit offsets
    (dict(M=64, K=1 << 21, segs=(128,)), _lib.OFT_EUNSUPPORTED),
])
def test_linear_size_range(kw, code):
    """The descriptor's sizes stay inside the kernels' index range: the
    launch grid's y limit for token tiles and 32-bit weight offsets."""
    d = _desc(**kw)
    n = C.c_size_t(0)
    assert _lib.load().oft_linear_workspace_bytes(C.byref(d), 1, C.byref(n)) == code


def test_linear_segment_sum_mismatch():
    d = _desc()
    d.N = 512
    n = C.c_size_t(0)
    assert _lib.load().oft_linear_workspace_bytes(C.byref(d), 1, C.byref(n)) == _lib.OFT_ESHAPE


def test_linear_null_and_misaligned_pointers_rejected():
    d = _desc()
    lib = _lib.load()
    assert lib.oft_linear_fwd(C.byref(d), None, None, None, None, None, None, 0, None) == _lib.OFT_EINVAL
    bad = C.c_void_p(0x1008)  # not 16-byte aligned
    ok = C.c_void_p(0x1000)
    assert lib.oft_linear_fwd(C.byref(d), bad, ok, ok, ok, ok, None, 0, None) == _lib.OFT_EINVAL
    # the reference-policy forward validates the same way (no R operand)
    assert lib.oft_linear_fwd_base(C.byref(d), None, ok, ok, ok, None, 0, None) == _lib.OFT_EINVAL
    assert lib.oft_linear_fwd_base(C.byref(d), ok, ok, bad, ok, None, 0, None) == _lib.OFT_EINVAL
    assert lib.oft_linear_fwd_base(C.byref(_desc(b=8)), ok, ok, ok, ok, None, 0, None) == _lib.OFT_EUNSUPPORTED
    assert lib.oft_linear_fwd_base(C.byref(_desc(M=0)), None, None, None, None, None, 0, None) == _lib.OFT_OK
    # dq requested with a too-small workspace
    nb = oft.oft_linear_workspace_bytes(d, oft.OFT_PASS_BWD)
    st = lib.oft_linear_bwd(C.byref(d), ok, ok, ok, ok, ok, ok, None, ok, ok, nb - 1, None)
    assert st == _lib.OFT_EWORKSPACE


def test_linear_workspace_query():
    d = _desc()
    assert oft.oft_linear_workspace_bytes(d, oft.OFT_PASS_FWD) == 0
    assert oft.oft_linear_workspace_bytes(d, oft.OFT_PASS_BWD) >= (384 // 32) * 1024 * 4
    with pytest.raises(oft.OftError):
        oft.oft_linear_workspace_bytes(d, 5)


@pytest.mark.parametrize("w_fmt,g", [(oft.OFT_W_FP8_E4M3, 0), (oft.OFT_W_INT4, 64)])
@pytest.mark.parametrize("M", [0, 1, 63, 64, 128, 129, 300, 4096])
@pytest.mark.parametrize("K,segs", [(128, (96, 32)), (256, (64,)), (320, (64, 64)), (2560, (4096, 1024, 1024)),
                                    (576, (320, 320)), (512, (256, 64, 96))])
def test_linear_bwd_workspace_covers_its_parts(w_fmt, g, M, K, segs):
    """Host-only backward planning over edge shapes (M = 0 included): the
    query succeeds and covers the dq partials, the rotated copy of dY for
    wide layers and, for wide layers with many tokens, the transposed weight
    (FP8 codes; INT4 with bf16 x and K % 256 == 0 reads its codes in place,
    so only fp32 x keeps a dequantised copy there)."""
    N = sum(segs)
    d = oft.linear_desc(M, K, segs, 32, oft.OFT_DT_BF16, w_fmt, g)
    nb = oft.oft_linear_workspace_bytes(d, oft.OFT_PASS_BWD)
    assert nb >= (N // 32) * 1024 * 4  # at least one slice of dq partials
    if K > 256 and M > 0:
        assert nb >= M * N * 2  # rotated dY
    if K > 256 and M > 128 and N % 64 == 0:
        if w_fmt == oft.OFT_W_INT4 and K % 256 == 0:
            d32 = oft.linear_desc(M, K, segs, 32, oft.OFT_DT_F32, w_fmt, g)
            nb32 = oft.oft_linear_workspace_bytes(d32, oft.OFT_PASS_BWD)
            assert nb32 >= nb + K * N * 2  # the bf16 copy: fp32 x only
        else:
            assert nb >= M * N * 2 + K * N * (1 if w_fmt == oft.OFT_W_FP8_E4M3 else 2)


def test_cayley_and_dequant_validation():
    lib = _lib.load()
    ok = C.c_void_p(0x1000)
    assert lib.cayley_build(ok, 4, 24, ok, None, None) == _lib.OFT_EUNSUPPORTED
    assert lib.cayley_build(ok, -1, 32, ok, None, None) == _lib.OFT_EINVAL
    assert lib.cayley_build(None, 0, 32, None, None, None) == _lib.OFT_OK  # empty no-op
    assert lib.oft_dequant(9, 4, 64, 32, ok, ok, ok, None) == _lib.OFT_EDTYPE
    assert lib.oft_dequant(0, 4, 60, 32, ok, ok, ok, None) == _lib.OFT_ESHAPE
    assert lib.oft_dequant(0, 4, 64, 48, ok, ok, ok, None) == _lib.OFT_EUNSUPPORTED
    assert lib.oft_dequant(0, 4, 64, 32, ok, None, ok, None) == _lib.OFT_EINVAL
    assert lib.oft_dequant(1, 0, 64, 0, None, None, None, None) == _lib.OFT_OK


def _moe(**kw):
    base = dict(T=128, E=16, k=4, H=256, I=128, g=32, b=32, chunk=4, renorm=0)
    base.update(kw)
    return oft.moe_desc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(k=17), _lib.OFT_EUNSUPPORTED),
    (dict(E=2048), _lib.OFT_EUNSUPPORTED),
    (dict(k=20, E=16), _lib.OFT_EUNSUPPORTED),
    (dict(b=64), _lib.OFT_EUNSUPPORTED),
    (dict(g=8), _lib.OFT_EUNSUPPORTED),
    (dict(H=200), _lib.OFT_ESHAPE),
    (dict(I=96), _lib.OFT_ESHAPE),
    (dict(chunk=0), _lib.OFT_EINVAL),
    (dict(renorm=2), _lib.OFT_EINVAL),
    (dict(T=-3), _lib.OFT_EINVAL),
    (dict(w_fmt=1), _lib.OFT_EDTYPE),  # FP8 experts are not a MoE format
    (dict(w_fmt=7), _lib.OFT_EDTYPE),
    (dict(w_fmt=2, g=0), _lib.OFT_OK),  # bf16 reference weights: no group
    (dict(w_fmt=2, g=0, I=96), _lib.OFT_ESHAPE),
    (dict(w_fmt=3), _lib.OFT_OK),  # FP4 experts
    (dict(w_fmt=3, g=0), _lib.OFT_EUNSUPPORTED),
    (dict(w_fmt=4, H=512, I=256), _lib.OFT_OK),  # tiled INT4: H, I multiples of 256
    (dict(w_fmt=4, H=384, I=256), _lib.OFT_ESHAPE),
    (dict(w_fmt=4, H=512, I=128), _lib.OFT_ESHAPE),
    (dict(w_fmt=4, H=512, I=256, g=16), _lib.OFT_EUNSUPPORTED),
])
def test_moe_validation(kw, code):
    d = _moe(**kw)
    n = C.c_size_t(0)
    assert _lib.load().oft_moe_workspace_bytes(C.byref(d), 0, C.byref(n)) == code


@pytest.mark.parametrize("kw,code", [
    (dict(T=262076, E=16, k=4), _lib.OFT_OK),            # ceil(T k / 16) + E = 65535
    (dict(T=262077, E=16, k=4), _lib.OFT_EUNSUPPORTED),  # 65536 work-list tiles along grid y
    (dict(H=1 << 17), _lib.OFT_EUNSUPPORTED),
    (dict(I=1 << 17), _lib.OFT_EUNSUPPORTED),
    (dict(H=1 << 16, I=(1 << 15) - 64), _lib.OFT_OK),      # I H < 2^31: 32-bit code offsets in an expert
    (dict(H=1 << 16, I=1 << 15), _lib.OFT_EUNSUPPORTED),
])
def test_moe_size_range(kw, code):
    d = _moe(**kw)
    n = C.c_size_t(0)
    assert _lib.load().oft_moe_workspace_bytes(C.byref(d), 0, C.byref(n)) == code


def test_slots_validation():
    lib = _lib.load()
    ok = C.c_void_p(0x1000)
    bad = C.c_void_p(0x1004)
    assert lib.oft_slots_switch(None, 0, 1, None) == _lib.OFT_EINVAL
    assert lib.oft_slots_switch(bad, 0, 1, None) == _lib.OFT_EINVAL
    assert lib.oft_slots_switch(ok, 2, 1, None) == _lib.OFT_EINVAL
    assert lib.oft_slots_switch(ok, -1, 1, None) == _lib.OFT_EINVAL
    d = _desc()
    args = [ok] * 8  # x, codes, scales, R_ops0, R_ops1, state, latch, y
    for i in range(8):
        a = list(args)
        a[i] = None
        assert lib.oft_linear_fwd_slots(C.byref(d), *a, None, 0, None) == _lib.OFT_EINVAL
        a[i] = bad
        assert lib.oft_linear_fwd_slots(C.byref(d), *a, None, 0, None) == _lib.OFT_EINVAL
    assert lib.oft_linear_fwd_slots(C.byref(_desc(b=8)), *args, None, 0, None) == _lib.OFT_EUNSUPPORTED
    # M == 0: only state and latch are needed
    a = [None] * 5 + [ok, None, None]
    assert lib.oft_linear_fwd_slots(C.byref(_desc(M=0)), *a, None, 0, None) == _lib.OFT_EINVAL


def test_moe_router_bwd_validation():
    lib = _lib.load()
    ok = C.c_void_p(0x1000)
    bad = C.c_void_p(0x1004)
    d = _moe()
    assert lib.oft_moe_router_bwd(C.byref(d), ok, ok, ok, None, None) == _lib.OFT_EINVAL
    assert lib.oft_moe_router_bwd(C.byref(d), ok, bad, ok, ok, None) == _lib.OFT_EINVAL
    assert lib.oft_moe_router_bwd(C.byref(_moe(k=17)), ok, ok, ok, ok, None) == _lib.OFT_EUNSUPPORTED
    assert lib.oft_moe_router_bwd(C.byref(_moe(T=0)), None, None, None, None, None) == _lib.OFT_OK


def test_moe_workspace_and_routing_checks():
    d = _moe()
    fwd = oft.oft_moe_workspace_bytes(d, oft.OFT_PASS_FWD)
    bwd = oft.oft_moe_workspace_bytes(d, oft.OFT_PASS_BWD)
    P = 128 * 4
    assert fwd >= P * 128 * 2 + P * 256 * 2  # act + down output
    assert bwd >= P * 256 * 2 + P * 256 * 2  # dH + dX per pair
    lib = _lib.load()
    rt = _lib.oft_moe_routing()  # all NULL
    ok = C.c_void_p(0x1000)
    assert lib.oft_moe_route(C.byref(d), ok, C.byref(rt), ok, fwd, None) == _lib.OFT_EINVAL


def test_moe_bf16_weights_need_no_scales():
    # bf16 reference weights: NULL scale pointers pass validation, which then
    # stops at the routing tables (all NULL here), before anything is enqueued
    lib = _lib.load()
    ok = C.c_void_p(0x1000)
    rt = _lib.oft_moe_routing()
    for w_fmt, code in ((oft.OFT_W_BF16, _lib.OFT_EINVAL), (oft.OFT_W_INT4, _lib.OFT_EINVAL)):
        d = _moe(w_fmt=w_fmt)
        assert lib.oft_moe_grouped_fwd(C.byref(d), ok, ok, ok, None, ok, None, ok, C.byref(rt), ok,
                                       ok, ok, 1 << 30, None) == code
    full = _lib.oft_moe_routing(*([0x1000] * 9))
    ws = oft.oft_moe_workspace_bytes(_moe(), oft.OFT_PASS_FWD)
    # INT4 without scales: rejected; bf16 without scales would launch, so only
    # the rejection is exercised here
    assert lib.oft_moe_grouped_fwd(C.byref(_moe()), ok, ok, ok, None, ok, None, ok, C.byref(full),
                                   ok, ok, ok, ws, None) == _lib.OFT_EINVAL


def test_prof_hook_without_gpu_work():
    """The timing hook's bookkeeping (no GPU needed while nothing is
    recorded): off by default, an empty list, and reads out of range
    rejected."""
    lib = _lib.load()
    assert lib.oft_prof_count() == 0
    buf = C.create_string_buffer(16)
    ms = C.c_float(0.0)
    assert lib.oft_prof_read(0, buf, 16, C.byref(ms)) == _lib.OFT_EINVAL
    assert lib.oft_prof_read(-1, buf, 16, C.byref(ms)) == _lib.OFT_EINVAL
    assert lib.oft_prof_enable(0) == _lib.OFT_OK  # stopping never touches the device
    assert lib.oft_prof_count() == 0


def test_every_gpu_test_shape_passes_validation():
    """Every dense and MoE configuration the GPU tests run is a valid
    descriptor (checked here on the CPU, so a bad test shape never reaches
    the GPU)."""
    import importlib.util

    from oft_inputs import CONFIGS

    def mod(name):
        spec = importlib.util.spec_from_file_location(name, os.path.join(os.path.dirname(__file__), name + ".py"))
        m = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(m)
        return m

    lib = _lib.load()
    dense_m, moe_m = mod("test_gpu_dense"), mod("test_gpu_moe")
    wf = {"int4": oft.OFT_W_INT4, "fp8": oft.OFT_W_FP8_E4M3, "fp4": oft.OFT_W_FP4_E2M1}
    dense = list(dense_m.SMALL.values()) + list(dense_m.FULL_EXTRA.values()) + \
        [c for c in CONFIGS.values() if hasattr(c, "segs")]
    n = C.c_size_t(0)
    for c in dense:
        d = oft.linear_desc(c.M, c.K, c.segs, c.b, oft.OFT_DT_F32 if c.x_dtype == "f32" else oft.OFT_DT_BF16,
                            wf[c.w_fmt], c.g)
        assert lib.oft_linear_workspace_bytes(C.byref(d), 1, C.byref(n)) == _lib.OFT_OK, c.name
    moe = list(moe_m.SMALL.values()) + list(moe_m.ROUTER.values()) + list(moe_m.MOE_FULL_FP4.values()) + \
        [c for c in CONFIGS.values() if not hasattr(c, "segs")]
    for c in moe:
        d = oft.moe_desc(c.T, c.E, c.k, c.H, c.I, c.g, c.b, c.chunk, 0, w_fmt=wf[c.w_fmt])
        assert lib.oft_moe_workspace_bytes(C.byref(d), 0, C.byref(n)) == _lib.OFT_OK, c.name
    for name in moe_m.TILED:
        c = moe_m.SMALL[name]
        d = oft.moe_desc(c.T, c.E, c.k, c.H, c.I, c.g, c.b, c.chunk, 0, w_fmt=oft.OFT_W_INT4_TILED)
        assert lib.oft_moe_workspace_bytes(C.byref(d), 0, C.byref(n)) == _lib.OFT_OK, name


def test_logprob_diff_and_moe_base_validation():
    lib = _lib.load()
    ok = C.c_void_p(0x1000)
    bad = C.c_void_p(0x1008)
    assert lib.oft_logprob_diff(0, 10, None, None, None, None, None) == _lib.OFT_OK  # no-op
    assert lib.oft_logprob_diff(-1, 10, ok, ok, ok, ok, None) == _lib.OFT_EINVAL
    assert lib.oft_logprob_diff(4, 0, ok, ok, ok, ok, None) == _lib.OFT_EINVAL
    assert lib.oft_logprob_diff(4, 10, ok, None, ok, ok, None) == _lib.OFT_EINVAL
    assert lib.oft_logprob_diff(4, 10, ok, ok, bad, ok, None) == _lib.OFT_EINVAL
    d = _moe()
    rt = oft.moe_routing(*([type("T", (), {"data_ptr": lambda self: 0x1000})()] * 9))
    args = (ok, ok, ok, ok, ok, ok, C.byref(rt), None, ok, ok, 1 << 30, None)
    assert lib.oft_moe_grouped_fwd_base(C.byref(_moe(b=64)), *args) == _lib.OFT_EUNSUPPORTED
    assert lib.oft_moe_grouped_fwd_base(C.byref(d), ok, ok, ok, ok, ok, ok, C.byref(rt), bad, ok, ok, 1 << 30,
                                        None) == _lib.OFT_EINVAL  # misaligned optional h
    assert lib.oft_moe_grouped_fwd_base(C.byref(d), ok, ok, ok, ok, ok, ok, C.byref(rt), None, None, ok, 1 << 30,
                                        None) == _lib.OFT_EINVAL  # y required
    assert lib.oft_moe_grouped_fwd_base(C.byref(d), ok, ok, ok, ok, ok, ok, C.byref(rt), None, ok, ok, 16,
                                        None) == _lib.OFT_EWORKSPACE


def test_noalloc_bwd_rejects_beyond_its_scratch_without_a_gpu():
    """The fixed-scratch backward refuses, before touching the device, a
    layer whose backward needs more than its array holds."""
    lib = _lib.load()
    ok = C.c_void_p(0x1000)
    big = _desc(M=8192, K=2560, segs=(9728, 9728), b=32, x_dtype=oft.OFT_DT_BF16, g=128)
    n = C.c_size_t(0)
    assert lib.oft_linear_workspace_bytes(C.byref(big), 1, C.byref(n)) == _lib.OFT_OK
    assert n.value > _lib.OFT_NOALLOC_SCRATCH_BYTES
    assert lib.oft_linear_bwd_noalloc(C.byref(big), ok, ok, ok, ok, ok, ok, ok, ok, None) == _lib.OFT_EWORKSPACE
    assert lib.oft_linear_bwd_noalloc(C.byref(_desc(b=8)), ok, ok, ok, ok, ok, ok, ok, ok, None) == \
        _lib.OFT_EUNSUPPORTED


def test_pack_int4_tiled_validation():
    """Host-side checks of oft_pack_int4_tiled (no GPU work: every call fails
    validation, or has nothing to do)."""
    lib = _lib.load()
    a, b, c, d = (C.c_void_p(0x10000 * i) for i in (1, 2, 3, 4))
    f = lib.oft_pack_int4_tiled
    assert f(0, 64, 128, 32, None, None, None, None, None) == _lib.OFT_OK  # nothing to pack
    assert f(1, 96, 128, 32, a, b, c, d, None) == _lib.OFT_ESHAPE    # rows % 64
    assert f(1, 64, 192, 64, a, b, c, d, None) == _lib.OFT_ESHAPE    # cols % 128
    assert f(1, 64, 128, 16, a, b, c, d, None) == _lib.OFT_EUNSUPPORTED
    assert f(-1, 64, 128, 32, a, b, c, d, None) == _lib.OFT_EINVAL
    assert f(1, 64, 128, 32, None, b, c, d, None) == _lib.OFT_EINVAL
    assert f(1, 64, 128, 32, C.c_void_p(0x10008), b, c, d, None) == _lib.OFT_EINVAL  # misaligned
    assert f(1, 64, 128, 32, a, b, C.c_void_p(0x10000 + 2048), d, None) == _lib.OFT_EINVAL  # codes overlap
    assert f(1, 64, 128, 32, a, b, c, C.c_void_p(0x20000 + 256), None) == _lib.OFT_EINVAL  # scales overlap
    assert f(1, 1 << 16, 1 << 16, 32, a, b, c, d, None) == _lib.OFT_EUNSUPPORTED  # 32-bit offsets
