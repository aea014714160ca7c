"""CPU checks of the C ABI: the library loads, exports every entry point that
include/gq.h declares, and rejects malformed arguments on the host before
anything is enqueued (no compute call is made here; no GPU is needed)."""

import ctypes
import os
import re

import pytest

import bit_grouped_moe_amd as gq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, NOT_SUPPORTED = 1, 801


def _declared():
    text = open(os.path.join(ROOT, "include", "gq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return gq.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(gq.EXPORTED_SYMBOLS) == names


def test_status_strings(lib):
    assert b"success" in lib.gq_status_string(0)
    assert b"InvalidValue" in lib.gq_status_string(INVALID)
    assert b"NotSupported" in lib.gq_status_string(NOT_SUPPORTED)


def test_route_max_tiles(lib):
    assert lib.gq_route_max_tiles(4096, 8, 128, 256) == 128 + 128 + 1
    assert lib.gq_route_max_tiles(16, 2, 4, 256) == 1 + 4 + 1
    assert lib.gq_route_max_tiles(0, 8, 128, 256) == 129
    assert lib.gq_route_max_tiles(-1, 8, 128, 256) == -1
    assert lib.gq_route_max_tiles(1, 8, 0, 256) == -1
    assert lib.gq_route_max_tiles(1, 8, 4, 0) == -1


F = ctypes.c_void_p(0x1000)          # a fake, aligned, never-dereferenced pointer
F2 = ctypes.c_void_p(0x1002)         # misaligned
NULL = None


def test_route_sort_rejects(lib):
    ok = dict(ids=F, rows=4, topk=2, E=8, tm=256, off=F, sp=F, tl=F, mt=11, nt=F)

    def call(**kw):
        a = {**ok, **kw}
        return lib.gq_route_sort(a["ids"], a["rows"], a["topk"], a["E"], a["tm"], a["off"],
                                 a["sp"], a["tl"], a["mt"], a["nt"], None)
    assert call(ids=NULL) == INVALID
    assert call(off=NULL) == INVALID
    assert call(rows=-1) == INVALID
    assert call(E=0) == INVALID
    assert call(tm=0) == INVALID
    assert call(mt=lib.gq_route_max_tiles(4, 2, 8, 256) - 1) == INVALID
    assert call(E=1025, mt=2000) == NOT_SUPPORTED


def test_decode_rejects(lib):
    assert lib.gq_nf4_decode(NULL, F, 4, 64, F, F, None) == INVALID
    assert lib.gq_nf4_decode(F, F, 4, 64, NULL, NULL, None) == INVALID
    assert lib.gq_nf4_decode(F, F, 4, 96, F, F, None) == INVALID
    assert lib.gq_nf4_decode(F, F, -1, 64, F, F, None) == INVALID
    assert lib.gq_nf4_decode(F, F, 4, 64, F2, NULL, None) == INVALID
    assert lib.gq_mxfp4_decode(F, F, 4, 48, F, F, None) == INVALID
    assert lib.gq_mxfp4_decode(F, NULL, 4, 32, F, F, None) == INVALID


def _gemv(lib, fn, **kw):
    a = dict(x=F, rows=1, K=2048, xs=2048, c=F, s=F, E=128, N=1536, ids=F, topk=8, ps=NULL,
             out=F)
    a.update(kw)
    return getattr(lib, fn)(a["x"], a["rows"], a["K"], a["xs"], a["c"], a["s"], a["E"], a["N"],
                            a["ids"], a["topk"], a["ps"], a["out"], None)


@pytest.mark.parametrize("fn", ["gq_nf4_grouped_gemv", "gq_mxfp4_grouped_gemv"])
def test_gemv_rejects(lib, fn):
    assert _gemv(lib, fn, x=NULL) == INVALID
    assert _gemv(lib, fn, ids=NULL) == INVALID
    assert _gemv(lib, fn, rows=0) == INVALID
    assert _gemv(lib, fn, rows=33) == NOT_SUPPORTED              # 33*8 pairs > 256
    assert _gemv(lib, fn, topk=0) == INVALID
    assert _gemv(lib, fn, K=2050, xs=2050) == INVALID
    assert _gemv(lib, fn, xs=2047) == INVALID
    assert _gemv(lib, fn, xs=2052) == INVALID
    assert _gemv(lib, fn, x=F2) == INVALID
    assert _gemv(lib, fn, rows=8, topk=33) == NOT_SUPPORTED
    assert _gemv(lib, fn, K=16384, xs=16384) == NOT_SUPPORTED
    assert _gemv(lib, fn, xs=1 << 31) == NOT_SUPPORTED            # 32-bit stride in the kernel
    if fn == "gq_nf4_grouped_gemv":
        assert _gemv(lib, fn, K=2080, xs=2080) == INVALID      # K % 64


def _gemm(lib, fn, **kw):
    a = dict(x=F, rows=4096, K=2048, xs=2048, c=F, s=F, E=128, N=1536, topk=8, ps=NULL,
             off=F, sp=F, tl=F, nt=F, mt=257, tm=256, out=F)
    a.update(kw)
    return getattr(lib, fn)(a["x"], a["rows"], a["K"], a["xs"], a["c"], a["s"], a["E"], a["N"],
                            a["topk"], a["ps"], a["off"], a["sp"], a["tl"], a["nt"], a["mt"],
                            a["tm"], a["out"], None)


@pytest.mark.parametrize("fn", ["gq_nf4_grouped_gemm", "gq_mxfp4_grouped_gemm"])
def test_gemm_rejects(lib, fn):
    assert _gemm(lib, fn, tl=NULL) == INVALID
    assert _gemm(lib, fn, rows=-1) == INVALID
    assert _gemm(lib, fn, N=1552) == INVALID                   # N % 32
    assert _gemm(lib, fn, mt=256) == INVALID                   # below the tile bound
    assert _gemm(lib, fn, out=F2) == INVALID
    assert _gemm(lib, fn, tm=128) == NOT_SUPPORTED
    assert _gemm(lib, fn, rows=0) == 0                         # nothing enqueued


def test_dgrad_rejects(lib):
    def call(**kw):
        a = dict(dy=F, P=16384, N=1536, ds=1536, c=F, s=F, E=128, K=2048, off=F, sp=F, tl=F,
                 nt=F, mt=193, tm=256, dx=F)
        a.update(kw)
        return lib.gq_nf4_grouped_dgrad(a["dy"], a["P"], a["N"], a["ds"], a["c"], a["s"],
                                        a["E"], a["K"], a["off"], a["sp"], a["tl"], a["nt"],
                                        a["mt"], a["tm"], a["dx"], None)
    assert call(dy=NULL) == INVALID
    assert call(N=1568, ds=1568) == INVALID                    # N % 64
    assert call(K=2080) == INVALID
    assert call(mt=100) == INVALID
    assert call(tm=64) == NOT_SUPPORTED
    assert call(P=0) == 0


def test_mxfp4_dgrad_rejects(lib):
    def call(**kw):
        a = dict(dy=F, P=8192, N=5760, ds=5760, c=F, s=F, E=32, K=2880, off=F, sp=F, tl=F,
                 nt=F, mt=65, tm=256, dx=F)
        a.update(kw)
        return lib.gq_mxfp4_grouped_dgrad(a["dy"], a["P"], a["N"], a["ds"], a["c"], a["s"],
                                          a["E"], a["K"], a["off"], a["sp"], a["tl"], a["nt"],
                                          a["mt"], a["tm"], a["dx"], None)
    assert call(s=NULL) == INVALID
    assert call(N=5792, ds=5792) == INVALID                    # N % 64
    assert call(K=2896) == INVALID                             # K % 32
    assert call(ds=5761) == INVALID                            # stride % 8
    assert call(mt=40) == INVALID
    assert call(tm=128) == NOT_SUPPORTED
    assert call(P=0) == 0


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(gq, "_lib", None)
    monkeypatch.setenv("GQ_LIBRARY", str(tmp_path / "nope.so"))
    with pytest.raises(gq.GQError):
        gq.load_library()


def test_probe_library_exports_its_header():
    """libgq_probes.so (the bench's control kernels) exports what
    include/gq_probes.h declares and rejects bad copy arguments on the host."""
    path = os.path.join(ROOT, "bit_grouped_moe_amd", "libgq_probes.so")
    if not os.path.exists(path):
        pytest.fail("libgq_probes.so is not built")
    text = open(os.path.join(ROOT, "include", "gq_probes.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(gq_probe_[a-z0-9_]+)\s*\(", text)))
    plib = ctypes.CDLL(path)
    assert names == ["gq_probe_copy", "gq_probe_empty", "gq_probe_mfma", "gq_probe_mfma_flops",
                     "gq_probe_mfma_per_wave_iter", "gq_probe_stream_read"]
    for n in names:
        assert hasattr(plib, n), n
    plib.gq_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_void_p]
    assert plib.gq_probe_copy(F, F, 24, None) == INVALID          # not a multiple of 16
    assert plib.gq_probe_copy(F2, F, 16, None) == INVALID         # misaligned source
    assert plib.gq_probe_copy(NULL, F, 16, None) == INVALID
    assert plib.gq_probe_copy(F, F, 0, None) == INVALID


def test_epilogue_entry_points_reject(lib):
    # SwiGLU GEMV: odd gate_up width, bad K
    assert lib.gq_nf4_grouped_gemv_swiglu(F, 1, 2048, 2048, F, F, 128, 1535, F, 8, F, None) == INVALID
    assert lib.gq_nf4_grouped_gemv_swiglu(F, 1, 2040, 2048, F, F, 128, 1536, F, 8, F, None) == INVALID
    assert lib.gq_nf4_grouped_gemv_swiglu(NULL, 1, 2048, 2048, F, F, 128, 1536, F, 8, F,
                                          None) == INVALID
    # SwiGLU GEMM: N % 64, tile_m
    assert lib.gq_nf4_grouped_gemm_swiglu(F, 4096, 2048, 2048, F, F, 128, 1568, 8, F, F, F, F,
                                          257, 256, F, None) == INVALID
    assert lib.gq_nf4_grouped_gemm_swiglu(F, 4096, 2048, 2048, F, F, 128, 1536, 8, F, F, F, F,
                                          257, 128, F, None) == NOT_SUPPORTED
    assert lib.gq_nf4_grouped_gemm_swiglu(F, 0, 2048, 2048, F, F, 128, 1536, 8, F, F, F, F,
                                          129, 256, F, None) == 0
    # down + combine: I % 64, too many pairs, I beyond one wave of segments
    assert lib.gq_nf4_grouped_gemv_down_combine(F, 1, 736, 736, F, F, 128, 2048, F, 8, NULL, F,
                                                None) == INVALID
    assert lib.gq_nf4_grouped_gemv_down_combine(F, 9, 768, 768, F, F, 128, 2048, F, 8, NULL, F,
                                                None) == NOT_SUPPORTED
    assert lib.gq_nf4_grouped_gemv_down_combine(F, 1, 4160, 4160, F, F, 128, 2048, F, 8, NULL, F,
                                                None) == NOT_SUPPORTED
    # two segments per lane (I > 2048) hold at most 32 pairs
    assert lib.gq_nf4_grouped_gemv_down_combine(F, 5, 4096, 4096, F, F, 128, 2048, F, 8, NULL, F,
                                                None) == NOT_SUPPORTED
    # MXFP4: I % 32, pairs, I limit, pair cap with two segments per lane
    assert lib.gq_mxfp4_grouped_gemv_down_combine(F, 1, 2870, 2880, F, F, 32, 2880, F, 4, NULL,
                                                  F, None) == INVALID
    assert lib.gq_mxfp4_grouped_gemv_down_combine(F, 17, 2880, 2880, F, F, 32, 2880, F, 4, NULL,
                                                  F, None) == NOT_SUPPORTED
    assert lib.gq_mxfp4_grouped_gemv_down_combine(F, 9, 2880, 2880, F, F, 32, 2880, F, 4, NULL,
                                                  F, None) == NOT_SUPPORTED
    assert lib.gq_mxfp4_grouped_gemv_down_combine(F, 1, 4128, 4128, F, F, 32, 2880, F, 4, NULL,
                                                  F, None) == NOT_SUPPORTED
    assert lib.gq_nf4_grouped_gemv_down_combine(F, 1, 768, 768, F, F, 128, 2048, F, 8, F2, F,
                                                None) == INVALID          # misaligned weights
    assert lib.gq_nf4_grouped_gemv_down_combine(F, 1, 768, 1 << 31, F, F, 128, 2048, F, 8, NULL,
                                                F, None) == NOT_SUPPORTED  # 32-bit stride
    # combine: H % 8, stride, rows == 0
    assert lib.gq_moe_combine(F, 4, 8, 2044, 2048, NULL, F, None) == INVALID
    assert lib.gq_moe_combine(F, 4, 8, 2048, 2040, NULL, F, None) == INVALID
    assert lib.gq_moe_combine(F2, 4, 8, 2048, 2048, NULL, F, None) == INVALID
    assert lib.gq_moe_combine(NULL, 0, 8, 2048, 2048, NULL, NULL, None) == 0


def test_gemv_pair_count_requires_matching_rows():
    """The decode GEMV wrappers take the pair count from topk_ids [rows, topk]
    and reject a topk_ids whose row count differs from x's (checked on the
    host, before any launch)."""
    import torch
    assert gq._gemv_pairs(torch.zeros((4, 8), dtype=torch.int32), 4) == 32
    for shape in ((3, 8), (5, 8), (32,), (4, 8, 1)):
        with pytest.raises(ValueError):
            gq._gemv_pairs(torch.zeros(shape, dtype=torch.int32), 4)


def test_scaled_mxfp4_entry_points_reject(lib):
    # split: K % 32, stride, null, misaligned output, rows == 0
    assert lib.gq_act_split_e4m3(F, 4, 48, 48, F, F, None) == INVALID
    assert lib.gq_act_split_e4m3(F, 4, 64, 60, F, F, None) == INVALID
    assert lib.gq_act_split_e4m3(NULL, 4, 64, 64, F, F, None) == INVALID
    assert lib.gq_act_split_e4m3(F, 4, 64, 64, F2, F, None) == INVALID
    assert lib.gq_act_split_e4m3(F, -1, 64, 64, F, F, None) == INVALID
    assert lib.gq_act_split_e4m3(F, 0, 64, 64, F, F, None) == 0
    # scaled GEMM: N % 32, K % 32, tile_m, max_tiles, null, 32-bit row offsets
    args = [F, F, 2048, 2880, F, F, 32, 5760, 4, NULL, F, F, F, F, 32 + 33 + 1, 256, F, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.gq_mxfp4_grouped_gemm_scaled(*a)
    assert call(a7=5750) == INVALID
    assert call(a3=2870) == INVALID
    assert call(a15=128) == NOT_SUPPORTED
    assert call(a14=60) == INVALID
    assert call(a0=NULL) == INVALID
    assert call(a1=F2) == INVALID
    assert call(a2=1 << 20, a14=(1 << 22) // 256 + 33 + 1) == NOT_SUPPORTED
    assert call(a2=0) == 0


def test_gpt_oss_activation_entry_points_reject(lib):
    """Host-side checks of the two entry points with the gpt-oss gated unit:
    the activation parameters, the gate_up width, and what the plain entry
    points already reject.  No kernel is launched."""
    nan, inf = float("nan"), float("inf")
    # GEMV: x, rows, K, stride, blocks, scales, E, N, ids, topk, alpha, limit, act
    g = [F, 1, 2880, 2880, F, F, 32, 5760, F, 4, 1.702, 7.0, F, None]

    def gemv(**kw):
        a = list(g)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.gq_mxfp4_grouped_gemv_swiglu(*a)
    assert gemv(a7=5761) == INVALID                        # odd gate_up width
    assert gemv(a11=-1.0) == INVALID
    assert gemv(a11=inf) == INVALID
    assert gemv(a10=nan) == INVALID
    assert gemv(a2=2870) == INVALID                        # K % 32
    assert gemv(a0=NULL) == INVALID
    assert gemv(a1=300) == NOT_SUPPORTED                   # > 256 pairs
    # scaled GEMM: codes, scales, rows, K, blocks, scales, E, N, topk, alpha,
    # limit, offsets, sorted, tiles, num_tiles, max_tiles, tile_m, act
    m = [F, F, 2048, 2880, F, F, 32, 5760, 4, 1.702, 7.0, F, F, F, F, 32 + 33 + 1, 256, F, None]

    def gemm(**kw):
        a = list(m)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.gq_mxfp4_grouped_gemm_scaled_swiglu(*a)
    assert gemm(a7=5750) == INVALID                        # N % 32
    assert gemm(a10=-0.5) == INVALID
    assert gemm(a9=inf) == INVALID
    assert gemm(a10=nan) == INVALID
    assert gemm(a16=128) == NOT_SUPPORTED
    assert gemm(a15=60) == INVALID
    assert gemm(a17=NULL) == INVALID
    assert gemm(a2=0) == 0
    # the same product written as the split: ..., act_codes, act_scales
    m2 = m[:17] + [F, F, None]

    def gemm_split(**kw):
        a = list(m2)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.gq_mxfp4_grouped_gemm_scaled_swiglu_split(*a)
    assert gemm_split(a7=5750) == INVALID                  # N % 32
    assert gemm_split(a7=5728) == NOT_SUPPORTED            # I = 2864: not whole 64-column steps
    assert gemm_split(a10=nan) == INVALID
    assert gemm_split(a17=NULL) == INVALID
    assert gemm_split(a18=NULL) == INVALID
    assert gemm_split(a17=ctypes.c_void_p(0x1008)) == INVALID   # codes not 16-byte aligned
    assert gemm_split(a18=ctypes.c_void_p(0x1002)) == INVALID   # scales not 4-byte aligned
    assert gemm_split(a16=128) == NOT_SUPPORTED
    assert gemm_split(a2=0) == 0


def test_host_bank_entry_points_reject_unpinned_memory(lib):
    """The host-resident GEMVs map the bank pointers before anything else:
    plain (unpinned) host memory and NULL are rejected, never launched on."""
    buf = ctypes.create_string_buffer(1 << 16)
    hp = ctypes.c_void_p(ctypes.addressof(buf))
    for fn in (lib.gq_nf4_grouped_gemv_host, lib.gq_mxfp4_grouped_gemv_host):
        assert fn(F, 1, 2048, 2048, hp, hp, 128, 1536, F, 8, NULL, F, None) == INVALID
        assert fn(F, 1, 2048, 2048, NULL, hp, 128, 1536, F, 8, NULL, F, None) == INVALID
        assert fn(F, 1, 2048, 2048, hp, NULL, 128, 1536, F, 8, NULL, F, None) == INVALID
