"""OFT dequant-GEMM for AMD Instinct MI355X (gfx950): Python binding.

Every function here marshals torch tensors (device memory) into the C ABI of
liboft.so (include/oft.h) and calls it on the current torch stream.  All
arithmetic runs in the library's HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C

from . import _lib
from ._lib import (OFT_DT_BF16, OFT_DT_F32, OFT_PASS_BWD, OFT_PASS_FWD, OFT_W_BF16,
                   OFT_W_FP4_E2M1, OFT_W_FP8_E4M3, OFT_W_INT4, OFT_W_INT4_TILED, OftError, oft_linear_desc,
                   oft_moe_desc, oft_moe_routing)

__all__ = [
    "OftError", "linear_desc", "moe_desc", "moe_routing", "cayley_build", "oft_dequant", "oft_pack_int4_tiled",
    "oft_linear_workspace_bytes", "oft_linear_fwd", "oft_linear_fwd_base", "oft_linear_bwd", "oft_linear_bwd_noalloc", "oft_logprob_diff",
    "oft_slots_switch", "oft_linear_fwd_slots",
    "oft_moe_workspace_bytes", "oft_moe_route", "oft_moe_router_bwd", "oft_moe_grouped_fwd", "oft_moe_grouped_fwd_base", "oft_moe_grouped_bwd", "abi_version",
    "prof_enable", "prof_records",
    "OFT_DT_BF16", "OFT_DT_F32", "OFT_W_INT4", "OFT_W_FP8_E4M3", "OFT_W_BF16", "OFT_W_FP4_E2M1", "OFT_W_INT4_TILED",
    "OFT_PASS_FWD",
    "OFT_PASS_BWD",
]


def _ptr(t):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return C.c_void_p(int(stream))
    import torch

    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def abi_version() -> int:
    return _lib.load().oft_abi_version()


def prof_enable(on: bool) -> None:
    """Start (clearing the list) or stop the library's per-step kernel timing."""
    _lib.check(_lib.load().oft_prof_enable(1 if on else 0), "oft_prof_enable")


def prof_records():
    """[(name, milliseconds)] of the recorded steps, in launch order (waits
    for each record's events)."""
    lib = _lib.load()
    out = []
    buf = C.create_string_buffer(64)
    ms = C.c_float(0.0)
    for i in range(lib.oft_prof_count()):
        _lib.check(lib.oft_prof_read(i, buf, 64, C.byref(ms)), "oft_prof_read")
        out.append((buf.value.decode(), float(ms.value)))
    return out


def linear_desc(M, K, segs, b, x_dtype=OFT_DT_BF16, w_fmt=OFT_W_INT4, g=0) -> oft_linear_desc:
    d = oft_linear_desc()
    d.M, d.K, d.N = int(M), int(K), int(sum(segs))
    d.x_dtype, d.w_fmt, d.g, d.b = int(x_dtype), int(w_fmt), int(g), int(b)
    d.n_seg = len(segs)
    for i, s in enumerate(segs):
        d.seg[i] = int(s)
    return d


def moe_desc(T, E, k, H, I, g, b, chunk, renorm=0, w_fmt=OFT_W_INT4) -> oft_moe_desc:
    d = oft_moe_desc()
    d.T, d.E, d.k, d.H, d.I, d.g, d.b, d.chunk, d.renorm, d.w_fmt = (
        int(v) for v in (T, E, k, H, I, g, b, chunk, renorm, w_fmt))
    return d


def moe_routing(topk_idx, topk_w, counts, offsets, perm, inv_perm, active, n_active,
                chunk_of_expert) -> oft_moe_routing:
    rt = oft_moe_routing()
    for name, t in (("topk_idx", topk_idx), ("topk_w", topk_w), ("counts", counts),
                    ("offsets", offsets), ("perm", perm), ("inv_perm", inv_perm),
                    ("active", active), ("n_active", n_active),
                    ("chunk_of_expert", chunk_of_expert)):
        setattr(rt, name, t.data_ptr())
    return rt


def cayley_build(q, nblk, b, R_f32, R_ops=None, stream=None):
    _lib.check(_lib.load().cayley_build(_ptr(q), nblk, b, _ptr(R_f32), _ptr(R_ops),
                                        _stream(stream)), "cayley_build")


def oft_dequant(w_fmt, rows, cols, g, codes, scales, out, stream=None):
    _lib.check(_lib.load().oft_dequant(w_fmt, rows, cols, g, _ptr(codes), _ptr(scales), _ptr(out),
                                       _stream(stream)), "oft_dequant")


def oft_pack_int4_tiled(count, rows, cols, g, codes, scales, codes_tiled, scales_tiled, stream=None):
    _lib.check(_lib.load().oft_pack_int4_tiled(count, rows, cols, g, _ptr(codes), _ptr(scales), _ptr(codes_tiled),
                                               _ptr(scales_tiled), _stream(stream)), "oft_pack_int4_tiled")


def oft_linear_workspace_bytes(desc, pass_) -> int:
    n = C.c_size_t(0)
    _lib.check(_lib.load().oft_linear_workspace_bytes(C.byref(desc), pass_, C.byref(n)),
               "oft_linear_workspace_bytes")
    return n.value


def oft_linear_fwd(desc, x, w_codes, w_scales, R_ops, y, ws=None, ws_bytes=0, stream=None):
    _lib.check(_lib.load().oft_linear_fwd(C.byref(desc), _ptr(x), _ptr(w_codes), _ptr(w_scales),
                                          _ptr(R_ops), _ptr(y), _ptr(ws), ws_bytes,
                                          _stream(stream)), "oft_linear_fwd")


def oft_linear_fwd_base(desc, x, w_codes, w_scales, y, ws=None, ws_bytes=0, stream=None):
    _lib.check(_lib.load().oft_linear_fwd_base(C.byref(desc), _ptr(x), _ptr(w_codes), _ptr(w_scales),
                                               _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
               "oft_linear_fwd_base")


def oft_slots_switch(state, slot, version, stream=None):
    _lib.check(_lib.load().oft_slots_switch(_ptr(state), int(slot), int(version), _stream(stream)),
               "oft_slots_switch")


def oft_linear_fwd_slots(desc, x, w_codes, w_scales, R_ops0, R_ops1, state, latch, y, ws=None, ws_bytes=0,
                         stream=None):
    _lib.check(_lib.load().oft_linear_fwd_slots(C.byref(desc), _ptr(x), _ptr(w_codes), _ptr(w_scales),
                                                _ptr(R_ops0), _ptr(R_ops1), _ptr(state), _ptr(latch), _ptr(y),
                                                _ptr(ws), ws_bytes, _stream(stream)),
               "oft_linear_fwd_slots")


def oft_linear_bwd(desc, dy, y_saved, w_codes, w_scales, R_f32, R_ops, dx=None, dq=None, ws=None,
                   ws_bytes=0, stream=None):
    _lib.check(_lib.load().oft_linear_bwd(C.byref(desc), _ptr(dy), _ptr(y_saved), _ptr(w_codes),
                                          _ptr(w_scales), _ptr(R_f32), _ptr(R_ops), _ptr(dx),
                                          _ptr(dq), _ptr(ws), ws_bytes, _stream(stream)),
               "oft_linear_bwd")


def oft_linear_bwd_noalloc(desc, dy, y_saved, w_codes, w_scales, R_f32, R_ops, dx=None, dq=None, stream=None):
    _lib.check(_lib.load().oft_linear_bwd_noalloc(C.byref(desc), _ptr(dy), _ptr(y_saved), _ptr(w_codes),
                                                  _ptr(w_scales), _ptr(R_f32), _ptr(R_ops), _ptr(dx), _ptr(dq),
                                                  _stream(stream)),
               "oft_linear_bwd_noalloc")


def oft_logprob_diff(logits_actor, logits_ref, labels, out, stream=None):
    T, V = logits_actor.shape
    _lib.check(_lib.load().oft_logprob_diff(int(T), int(V), _ptr(logits_actor), _ptr(logits_ref), _ptr(labels),
                                            _ptr(out), _stream(stream)), "oft_logprob_diff")


def oft_moe_workspace_bytes(desc, pass_) -> int:
    n = C.c_size_t(0)
    _lib.check(_lib.load().oft_moe_workspace_bytes(C.byref(desc), pass_, C.byref(n)),
               "oft_moe_workspace_bytes")
    return n.value


def oft_moe_route(desc, logits, rt, ws, ws_bytes, stream=None):
    _lib.check(_lib.load().oft_moe_route(C.byref(desc), _ptr(logits), C.byref(rt), _ptr(ws),
                                         ws_bytes, _stream(stream)), "oft_moe_route")


def oft_moe_router_bwd(desc, logits, topk_idx, dw, d_logits, stream=None):
    _lib.check(_lib.load().oft_moe_router_bwd(C.byref(desc), _ptr(logits), _ptr(topk_idx), _ptr(dw),
                                              _ptr(d_logits), _stream(stream)), "oft_moe_router_bwd")


def oft_moe_grouped_fwd(desc, x, logits, wgu_codes, wgu_scales, wd_codes, wd_scales, R_ops, rt,
                        h_saved, y, ws, ws_bytes, stream=None):
    _lib.check(_lib.load().oft_moe_grouped_fwd(
        C.byref(desc), _ptr(x), _ptr(logits), _ptr(wgu_codes), _ptr(wgu_scales), _ptr(wd_codes),
        _ptr(wd_scales), _ptr(R_ops), C.byref(rt), _ptr(h_saved), _ptr(y), _ptr(ws), ws_bytes,
        _stream(stream)), "oft_moe_grouped_fwd")


def oft_moe_grouped_fwd_base(desc, x, logits, wgu_codes, wgu_scales, wd_codes, wd_scales, rt, h=None, y=None,
                             ws=None, ws_bytes=0, stream=None):
    _lib.check(_lib.load().oft_moe_grouped_fwd_base(
        C.byref(desc), _ptr(x), _ptr(logits), _ptr(wgu_codes), _ptr(wgu_scales), _ptr(wd_codes), _ptr(wd_scales),
        C.byref(rt), _ptr(h), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)), "oft_moe_grouped_fwd_base")


def oft_moe_grouped_bwd(desc, dy, rt, h_saved, wgu_codes, wgu_scales, wd_codes, wd_scales, R_f32,
                        R_ops, dx=None, dq=None, dw=None, ws=None, ws_bytes=0, stream=None):
    _lib.check(_lib.load().oft_moe_grouped_bwd(
        C.byref(desc), _ptr(dy), C.byref(rt), _ptr(h_saved), _ptr(wgu_codes), _ptr(wgu_scales),
        _ptr(wd_codes), _ptr(wd_scales), _ptr(R_f32), _ptr(R_ops), _ptr(dx), _ptr(dq), _ptr(dw),
        _ptr(ws), ws_bytes, _stream(stream)), "oft_moe_grouped_bwd")
