"""C-ABI contract of libmoe.so, checked without a GPU.

The library must load, export every entry point include/moe.h declares, and
reject every invalid or unsupported argument on the host before anything is
enqueued (so none of these calls touches the device; fake but aligned
addresses are enough).
"""
import ctypes
import os
import re

import pytest

import sparse_moe_layer_gemm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVAL, UNSUP, WS_SMALL = 0, 1, 2, 3
A = 0x10000  # fake 16-byte aligned device addresses (never dereferenced)
B, C, D, F, G, Hh, J = (A * i for i in range(2, 9))
MIS = A + 4  # misaligned


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    lib = moe.load_library()
    names = header_functions()
    assert set(names) == set(moe.ENTRY_POINTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = moe.load_library()
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE_TOO_SMALL"
    assert lib.moe_status_string(99) == b"MOE_ERR_UNKNOWN"


def _w(dtype=1, gu=A, dn=B, gus=None, dns=None, gug=None, dng=None, qmode=0):
    return moe.CExpertWeights(dtype, qmode, gu, dn, gus, dns, gug, dng)


def route(**kw):
    a = dict(x=A, x_dt=1, T=128, H=5120, wr=B, bias=None, E=256, k=8, l_dt=1, logits=C,
             logits_f32=None, ids=D, w=F, ws=G, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return moe.load_library().moe_route(*a.values())


def test_route_validation():
    assert route(T=0, x=None, wr=None, ids=None, w=None, ws=None) == OK  # no-op
    assert route(k=9) == UNSUP
    assert route(E=257) == UNSUP
    assert route(k=0) == INVAL
    assert route(k=5, E=4) == INVAL
    assert route(T=-1) == INVAL
    assert route(H=5000) == UNSUP
    assert route(x_dt=2) == INVAL
    assert route(l_dt=0) == UNSUP  # fp32 logits need fp32 x
    assert route(l_dt=7) == INVAL
    assert route(x=None) == INVAL
    assert route(ids=None) == INVAL
    assert route(x=MIS) == INVAL
    assert route(ws_bytes=16) == WS_SMALL
    assert route(T=(1 << 31) // 8) == UNSUP
    assert route(T=1 << 24, k=1) == UNSUP  # token limit


def test_route_workspace_size_positive():
    lib = moe.load_library()
    assert lib.moe_route_workspace_size(128, 5120, 256) >= 128 * 256 * 4
    assert lib.moe_route_workspace_size(0, 5120, 256) == 0


def permute(**kw):
    a = dict(ids=A, T=128, k=8, E=256, counts=B, offsets=C, sp=D, pp=F, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return moe.load_library().moe_permute(*a.values())


def test_permute_validation():
    assert permute(T=0, ids=None, sp=None, pp=None) == OK
    assert permute(k=9) == UNSUP
    assert permute(E=300) == UNSUP
    assert permute(k=0) == INVAL
    assert permute(counts=None) == INVAL
    assert permute(sp=MIS) == INVAL


def experts(w=None, **kw):
    w = w if w is not None else _w()
    a = dict(x=A, x_dt=1, T=128, H=5120, I=1536, E=256, k=8, offsets=B, sp=C, w=ctypes.byref(w),
             y=D, ws=F, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return moe.load_library().moe_experts(*a.values())


def test_experts_validation():
    assert experts(T=0, x=None, offsets=None, sp=None, y=None, ws=None) == OK
    assert experts(I=100) == UNSUP
    assert experts(I=0) == INVAL
    assert experts(w=_w(dtype=0)) == UNSUP  # fp32 weights need fp32 x
    assert experts(w=_w(dtype=1), x_dt=0) == UNSUP
    assert experts(w=_w(dtype=5)) == INVAL
    assert experts(w=_w(dtype=2)) == INVAL  # FP8 needs channel scales
    assert experts(w=_w(dtype=3, gus=G, dns=Hh)) == INVAL  # FP4 needs global scales
    assert experts(w=_w(gu=None)) == INVAL
    assert experts(w=_w(gu=MIS)) == INVAL
    assert experts(ws_bytes=1) == WS_SMALL
    assert moe.load_library().moe_experts(A, 1, 8, 64, 64, 8, 2, B, C, None, D, F, 1 << 30, None) == INVAL


def test_permute_workspace():
    lib = moe.load_library()
    assert lib.moe_permute_workspace_size(2048, 8, 256) == 0  # one workgroup up to 16384 pairs
    big = lib.moe_permute_workspace_size(16384, 8, 256)
    assert big >= 256 * (131072 // 4096) * 4  # per-segment histograms
    assert permute(T=16384, k=8, E=256, ws=None, ws_bytes=0) == INVAL
    assert permute(T=16384, k=8, E=256, ws=G, ws_bytes=big - 1) == WS_SMALL


def test_experts_qmode_validation():
    fp4 = dict(dtype=3, gus=G, dns=Hh, gug=A, dng=B)
    assert experts(w=_w(qmode=7)) == INVAL
    assert experts(w=_w(dtype=1, qmode=1)) == UNSUP  # fp8-MFMA mode is for quantised weights
    assert experts(w=_w(**fp4, qmode=1), I=4160) == UNSUP  # h block scales: I <= 4096
    assert experts(w=_w(**fp4, qmode=1), T=0, x=None, offsets=None, sp=None, y=None, ws=None) == OK
    lib = moe.load_library()
    ww, w8 = _w(**fp4), _w(**fp4, qmode=1)
    sw = lib.moe_experts_workspace_size(4096, 5120, 1536, 256, 8, ctypes.byref(ww))
    s8 = lib.moe_experts_workspace_size(4096, 5120, 1536, 256, 8, ctypes.byref(w8))
    # the fp8 mode adds E4M3 x [T, H], per-token scales, E4M3 h [T*k, I] and block scales
    assert s8 >= sw + 4096 * 5120 + 4096 * 4 + 4096 * 8 * 1536 + 4096 * 8 * 12


def test_experts_workspace_size():
    lib = moe.load_library()
    w = _w()
    assert lib.moe_experts_workspace_size(128, 5120, 1536, 256, 8, ctypes.byref(w)) >= 1024 * 1536 * 2
    w32 = _w(dtype=0)
    assert lib.moe_experts_workspace_size(64, 512, 256, 32, 4, ctypes.byref(w32)) >= 256 * 256 * 4


def finalize(**kw):
    a = dict(y=A, pp=B, w=C, T=128, k=8, H=5120, out_dt=1, out=D, out_f32=None, stream=None)
    a.update(kw)
    return moe.load_library().moe_finalize(*a.values())


def test_finalize_validation():
    assert finalize(T=0, y=None, pp=None, w=None, out=None) == OK
    assert finalize(k=9) == UNSUP
    assert finalize(H=100) == UNSUP
    assert finalize(out_dt=2) == INVAL
    assert finalize(out=None) == INVAL
    assert finalize(out_f32=MIS) == INVAL


def experts_rows16(w=None, **kw):
    w = w if w is not None else _w()
    a = dict(x=A, x_dt=1, T=16384, H=5120, I=1536, E=256, k=8, off=B, sp=C, w=ctypes.byref(w),
             y16=D, ysc=F, ws=G, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return moe.load_library().moe_experts_rows16(*a.values())


def test_experts_rows16_validation():
    assert experts_rows16(T=0, x=None, off=None, sp=None, y16=None, ysc=None, ws=None) == OK
    assert experts_rows16(T=128) == UNSUP  # 4 rows per expert: the streaming kernels
    assert experts_rows16(T=128, w=_w(dtype=2, gus=G, dns=Hh)) == UNSUP  # FP8, streaming sizes
    # NVFP4 streams up to 16 rows per expert (T*k = 16 E here), FP8 up to 31
    fp4 = _w(dtype=3, gus=G, dns=Hh, gug=J, dng=J)
    assert experts_rows16(T=512, w=fp4) == UNSUP
    assert experts_rows16(T=1000, w=_w(dtype=2, gus=G, dns=Hh)) == UNSUP
    assert experts_rows16(ysc=None) == INVAL
    assert experts_rows16(y16=MIS) == INVAL
    assert experts_rows16(ws_bytes=1024) == WS_SMALL
    assert experts_rows16(k=9) == UNSUP


def finalize_rows16(**kw):
    a = dict(y16=A, ysc=B, pp=C, w=D, T=128, k=8, H=5120, out_dt=1, out=F, out_f32=None,
             stream=None)
    a.update(kw)
    return moe.load_library().moe_finalize_rows16(*a.values())


def test_tiled_work_lists_that_overflow_are_unsupported():
    # H = 2^30: the down GEMM's work list would pass 2^30 items
    assert experts_rows16(H=1 << 30) == UNSUP
    assert experts(H=1 << 30, T=16384) == UNSUP


def test_finalize_rows16_validation():
    assert finalize_rows16(T=0, y16=None, ysc=None, pp=None, w=None, out=None) == OK
    assert finalize_rows16(k=9) == UNSUP
    assert finalize_rows16(H=100) == UNSUP
    assert finalize_rows16(out_dt=2) == INVAL
    assert finalize_rows16(ysc=None) == INVAL
    assert finalize_rows16(out_f32=MIS) == INVAL


def finalize_norm(**kw):
    a = dict(y=A, pp=B, w=C, T=128, k=8, H=5120, res=D, gp=F, gn=G, eps=1e-6, res_out=D,
             normed=Hh, stream=None)
    a.update(kw)
    return moe.load_library().moe_finalize_norm(*a.values())


def test_finalize_norm_validation():
    assert finalize_norm(T=0, y=None, pp=None, w=None, res=None, gp=None, gn=None, res_out=None,
                         normed=None) == OK
    assert finalize_norm(k=9) == UNSUP
    assert finalize_norm(H=100) == UNSUP
    assert finalize_norm(H=16384 + 64) == UNSUP
    assert finalize_norm(eps=-1.0) == INVAL
    assert finalize_norm(eps=float("nan")) == INVAL
    assert finalize_norm(eps=float("inf")) == INVAL
    assert finalize_norm(gn=None) == INVAL
    assert finalize_norm(res=MIS) == INVAL
    assert finalize_norm(normed=D) == INVAL  # normed may not alias the residual
    assert finalize_norm(k=0) == INVAL


# fake addresses far enough apart that [T, H] bf16 rows at them do not overlap
R1, R2, R3 = 1 << 32, 2 << 32, 3 << 32
ROWS = 128 * 5120 * 2


def test_finalize_norm_rejects_overlapping_outputs():
    ok = dict(res=R1, res_out=R1, normed=R2)
    assert finalize_norm(**{**ok, "normed": R1 + ROWS - 16}) == INVAL  # normed inside residual
    assert finalize_norm(**{**ok, "normed": R1 - ROWS + 16}) == INVAL  # normed ends inside it
    assert finalize_norm(res=R1, res_out=R2, normed=R2 + 4096) == INVAL  # inside residual_out
    assert finalize_norm(res=R1, res_out=R1 + 4096, normed=R2) == INVAL  # partial in-place


def finalize_norm_rows16(**kw):
    a = dict(y16=A, ysc=B, pp=C, w=D, T=128, k=8, H=5120, res=R1, gp=F, gn=G, eps=1e-6,
             res_out=R1, normed=R2, stream=None)
    a.update(kw)
    return moe.load_library().moe_finalize_norm_rows16(*a.values())


def test_finalize_norm_rows16_validation():
    assert finalize_norm_rows16(T=0, y16=None, ysc=None, pp=None, w=None, res=None, gp=None,
                                gn=None, res_out=None, normed=None) == OK
    assert finalize_norm_rows16(k=9) == UNSUP
    assert finalize_norm_rows16(H=100) == UNSUP
    assert finalize_norm_rows16(H=16384 + 64) == UNSUP
    assert finalize_norm_rows16(eps=float("nan")) == INVAL
    assert finalize_norm_rows16(y16=None) == INVAL
    assert finalize_norm_rows16(ysc=MIS) == INVAL
    assert finalize_norm_rows16(normed=R1 + 64) == INVAL
    assert finalize_norm_rows16(res_out=R2 + 64) == INVAL


def forward_norm(w=None, **kw):
    w = w if w is not None else _w()
    a = dict(x=A, T=128, H=5120, I=1536, E=256, k=8, wr=B, bias=None, w=ctypes.byref(w),
             res=R1, gp=F, gn=G, eps=1e-6, res_out=R1, normed=R2, logits=None, ids=None, tw=None,
             ws=R3, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return moe.load_library().moe_forward_norm(*a.values())


def test_forward_norm_validation():
    assert forward_norm(T=0, x=None, wr=None, res=None, gp=None, gn=None, res_out=None,
                        normed=None, ws=None) == OK
    assert forward_norm(k=9) == UNSUP
    assert forward_norm(H=16384 + 64) == UNSUP
    assert forward_norm(w=_w(dtype=0)) == UNSUP  # fp32 experts need fp32 x
    assert forward_norm(x=None) == INVAL
    assert forward_norm(res_out=None) == INVAL
    assert forward_norm(gp=MIS) == INVAL
    assert forward_norm(eps=-1.0) == INVAL
    assert forward_norm(normed=R1 + 64) == INVAL
    assert forward_norm(ws=None) == INVAL
    assert forward_norm(ws_bytes=1024) == WS_SMALL


def forward(w=None, **kw):
    w = w if w is not None else _w()
    a = dict(x=A, x_dt=1, T=128, H=5120, I=1536, E=256, k=8, wr=B, bias=None, w=ctypes.byref(w),
             out_dt=1, out=C, out_f32=None, l_dt=1, logits=None, ids=None, tw=None, ws=D,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return moe.load_library().moe_forward(*a.values())


def test_forward_validation():
    assert forward(T=0, x=None, wr=None, out=None, ws=None) == OK
    assert forward(k=9) == UNSUP
    assert forward(E=4, k=8) == INVAL
    assert forward(out_dt=3) == INVAL
    assert forward(l_dt=0) == UNSUP
    assert forward(out=None) == INVAL
    assert forward(ids=MIS) == INVAL
    assert forward(ws_bytes=1024) == WS_SMALL
    assert forward(ws=None) == INVAL
    assert forward(ws=MIS) == INVAL
    assert forward(w=_w(dtype=3, gus=G, dns=Hh, gug=J, dng=None)) == INVAL
    assert forward(w=_w(dtype=3, gus=G, dns=Hh, gug=J, dng=J), x_dt=0, l_dt=0) == UNSUP


def forward_noalloc(w=None, **kw):
    w = w if w is not None else _w()
    a = dict(x=A, x_dt=1, T=128, H=5120, I=1536, E=256, k=8, wr=B, bias=None, w=ctypes.byref(w),
             out_dt=1, out=C, out_f32=None, l_dt=1, logits=None, ids=None, tw=None, stream=None)
    a.update(kw)
    return moe.load_library().moe_forward_noalloc(*a.values())


def test_forward_noalloc_validation():
    """Every rejection happens on the host, before the scratch area is looked up."""
    assert forward_noalloc(T=0, x=None, wr=None, out=None) == OK
    assert forward_noalloc(k=9) == UNSUP
    assert forward_noalloc(E=4, k=8) == INVAL
    assert forward_noalloc(out=None) == INVAL
    assert forward_noalloc(x=MIS) == INVAL
    assert forward_noalloc(ids=MIS) == INVAL
    assert forward_noalloc(w=_w(dtype=3, gus=G, dns=Hh, gug=J, dng=None)) == INVAL
    # beyond the scratch area: a prefill-sized call is rejected with a clear status
    assert forward_noalloc(T=16384) == WS_SMALL
    assert forward_noalloc(T=512, I=2560) == WS_SMALL


def test_forward_noalloc_limit_covers_decode():
    """64 MiB holds the whole decode layer's workspace up to T = 128 (I <= 2560, every
    weight format), and the limit is exactly where moe_forward's workspace exceeds it."""
    lib = moe.load_library()
    cap = moe.NOALLOC_SCRATCH_BYTES
    for w in (_w(), _w(dtype=2, gus=G, dns=Hh), _w(dtype=3, gus=G, dns=Hh, gug=J, dng=J),
              _w(dtype=3, gus=G, dns=Hh, gug=J, dng=J, qmode=1)):
        for I in (1536, 2560):
            for T in (1, 2, 8, 32, 128):
                assert lib.moe_forward_workspace_size(T, 5120, I, 256, 8, ctypes.byref(w)) <= cap
    w = _w()
    T = 128
    while lib.moe_forward_workspace_size(T, 5120, 1536, 256, 8, ctypes.byref(w)) <= cap:
        T += 1
    assert forward_noalloc(T=T) == WS_SMALL


def test_forward_workspace_covers_stages():
    lib = moe.load_library()
    w = _w()
    T, H, I, E, k = 128, 5120, 1536, 256, 8
    fw = lib.moe_forward_workspace_size(T, H, I, E, k, ctypes.byref(w))
    assert fw >= T * k * H * 4 + lib.moe_experts_workspace_size(T, H, I, E, k, ctypes.byref(w))


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        moe_mod = moe
        saved = moe_mod._lib
        try:
            moe_mod._lib = None
            moe_mod.load_library(str(tmp_path / "missing.so"))
        finally:
            moe_mod._lib = saved


def test_hbm_read_validation():
    f = moe.load_library().moe_hbm_read
    assert f(A, 0, B, None) == OK  # nothing to read: no launch
    assert f(None, 16, B, None) == INVAL
    assert f(A, 16, None, None) == INVAL
    assert f(MIS, 16, B, None) == INVAL
    assert f(A, 24, B, None) == INVAL
