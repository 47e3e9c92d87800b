"""C-ABI boundary checks that need no GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import fp8_kv_cache_sparse_amd as smqa
from fp8_kv_cache_sparse_amd._binding import Layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smqa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(smqa.LIB_PATH), reason="libsmqa.so not built")

A16 = 0x100000          # fake, suitably aligned device addresses: never dereferenced by validation
A4 = 0x200004


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)) -
                  {"if", "while", "for", "return", "sizeof"})


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("sparse_mqa_score", "topk_select", "sparse_mqa_attend", "sparse_mqa_attend_fp8kv",
              "sparse_mqa_attend_nvfp4", "sparse_mqa_attend_fused", "smqa_attend_fused_workspace_size",
              "sparse_mqa_attend_mxfp8q",
              "decode_step_fused", "decode_step_noalloc",
              "decode_step",
              "smqa_topk_workspace_size", "smqa_attend_workspace_size",
              "smqa_decode_step_workspace_size", "smqa_attend_plan", "smqa_last_error", "smqa_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(smqa.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def layout(B=1, T=1, max_ctx=8192, seq=A16, qs=A4, qp=A4):
    return Layout(B, seq, T, qs, qp, max_ctx)


def lib():
    return smqa.load()


def err():
    return lib().smqa_last_error().decode()


def score(L, **kw):
    a = dict(q=A16, w=A4, k=A16, ks=None, cand=None, n_cand=0, Hi=64, Di=128, s=A4, ld=8192)
    a.update(kw)
    return lib().sparse_mqa_score(ctypes.byref(L) if L is not None else None, a["q"], a["w"], a["k"],
                                  a["ks"], a["cand"], a["n_cand"], a["Hi"], a["Di"], a["s"], a["ld"], None)


def test_score_validation():
    L = layout()
    assert score(None) == -1 and "layout" in err()
    assert score(L, q=None) == -1 and "q_fp8" in err()
    assert score(L, s=None) == -1
    assert score(L, Di=96) == -4 and "Di" in err()
    assert score(L, Hi=0) == -4 and score(L, Hi=129) == -4
    assert score(L, ld=100) == -2 and "ld_scores" in err()
    assert score(L, q=A16 + 8) == -3 and "aligned" in err()
    assert score(L, cand=A4, n_cand=0) == -2
    assert score(L, cand=A4, n_cand=300, ld=200) == -2
    assert score(layout(B=0)) == -2
    assert score(layout(T=-1)) == -2
    assert score(layout(seq=None)) == -1
    assert score(layout(seq=A16 + 4)) == -3
    assert score(layout(max_ctx=0)) == -2
    # zero queries: nothing to do, no launch
    assert score(layout(T=0)) == 0


def topk(L, k=2048, ws=None, nbytes=0, **kw):
    a = dict(s=A4, ld=8192, cand=None, n_cand=0, idx=A4, val=None)
    a.update(kw)
    return lib().topk_select(ctypes.byref(L), a["s"], a["ld"], a["cand"], a["n_cand"], k, a["idx"],
                             a["val"], ws, nbytes, None)


def test_topk_validation_and_workspace():
    L = layout()
    assert topk(L, k=0) == -4 and topk(L, k=4097) == -4
    assert topk(L, idx=None) == -1
    assert topk(L, val=A4 + 2) == -3 and "val" in err()
    assert topk(L, ld=10) == -2
    big = layout(max_ctx=100000)
    need = lib().smqa_topk_workspace_size(ctypes.byref(big), 2048, 0)
    assert need > 0
    assert topk(big, ld=100000) == -5 and "workspace" in err()
    assert topk(big, ld=100000, ws=A16 * 16, nbytes=need - 1) == -5
    assert topk(big, ld=100000, ws=A16 * 16 + 16, nbytes=need) == -3
    # short rows need no workspace
    assert lib().smqa_topk_workspace_size(ctypes.byref(L), 2048, 0) == 0


def attend(L, **kw):
    a = dict(q=A16, c=A16, e=A4, rs=None, idx=A4, k=2048, swa=A16, ss=None, p0=A4, clip=None, W=128,
             Hq=64, D=1664, sc=0.0245, out=A16, lse=None, ws=None, nb=0)
    a.update(kw)
    return lib().sparse_mqa_attend(ctypes.byref(L), a["q"], a["c"], a["e"], a["rs"], a["idx"], a["k"],
                                   a["swa"], a["ss"], a["p0"], a["clip"], a["W"], a["Hq"], a["D"], a["sc"],
                                   a["out"], a["lse"], a["ws"], a["nb"], None)


def test_attend_validation():
    L = layout()
    assert attend(L, D=1600) == -4 and "D" in err()
    assert attend(L, D=4096) == -4
    assert attend(L, Hq=24) == -4 and attend(L, Hq=256) == -4
    assert attend(L, W=0) == -4 and attend(L, W=129) == -4
    assert attend(L, k=0) == -4
    assert attend(L, swa=None) == -1 and attend(L, p0=None) == -1 and attend(L, idx=None) == -1
    assert attend(L, out=A16 + 4) == -3
    assert attend(L, sc=float("nan")) == -2
    # one decode query needs split-KV partials -> workspace required
    need = lib().smqa_attend_workspace_size(ctypes.byref(L), 2048, 128, 64, 1664)
    assert need > 0
    assert attend(L) == -5
    assert attend(layout(T=0)) == 0


def attend8(L, **kw):
    a = dict(q=A16, c=A16, rs=None, idx=A4, k=2048, swa=A16, ss=None, p0=A4, clip=None, W=128,
             Hq=64, D=1664, sc=0.0245, out=A16, lse=None, ws=None, nb=0)
    a.update(kw)
    return lib().sparse_mqa_attend_fp8kv(ctypes.byref(L), a["q"], a["c"], a["rs"], a["idx"], a["k"],
                                         a["swa"], a["ss"], a["p0"], a["clip"], a["W"], a["Hq"],
                                         a["D"], a["sc"], a["out"], a["lse"], a["ws"], a["nb"], None)


def test_attend_fp8kv_validation():
    L = layout()
    assert attend8(L, Hq=48) == -4 and "Hq" in err()        # only 32-head groups
    assert attend8(L, D=1792) == -4 and attend8(L, D=1600) == -4
    assert attend8(L, c=None) == -1 and attend8(L, idx=None) == -1
    assert attend8(L, c=A16 + 4) == -3
    assert attend8(L, k=5000) == -4 and attend8(L, W=0) == -4
    assert attend8(L) == -5                                  # split partials need the workspace
    assert attend8(layout(T=0)) == 0


def attend_nv(L, **kw):
    a = dict(q=A16, c=A16, s=A4, rs=None, g=1.0, idx=A4, k=2048, swa=A16, ss=None, p0=A4, clip=None,
             W=128, Hq=64, D=1664, sc=0.0245, out=A16, lse=None, ws=None, nb=0)
    a.update(kw)
    return lib().sparse_mqa_attend_nvfp4(ctypes.byref(L), a["q"], a["c"], a["s"], a["rs"], a["g"],
                                         a["idx"], a["k"], a["swa"], a["ss"], a["p0"], a["clip"],
                                         a["W"], a["Hq"], a["D"], a["sc"], a["out"], a["lse"], a["ws"],
                                         a["nb"], None)


def test_attend_nvfp4_validation():
    L = layout()
    assert attend_nv(L, Hq=48) == -4 and "Hq" in err()
    assert attend_nv(L, D=1792) == -4
    assert attend_nv(L, s=None) == -1 and attend_nv(L, c=None) == -1
    assert attend_nv(L, s=A4 + 2) == -3 and attend_nv(L, c=A16 + 4) == -3
    assert attend_nv(L, g=0.0) == -2 and attend_nv(L, g=float("nan")) == -2
    assert attend_nv(L, g=float("inf")) == -2 and attend_nv(L, g=-1.0) == -2
    assert attend_nv(L, g=1e-31) == -2 and attend_nv(L, g=2e30) == -2
    assert attend_nv(L) == -5
    assert attend_nv(layout(T=0)) == 0


def attend_fused(L, **kw):
    a = dict(q=A16, rc=A16, rs_=A16, R=32, c=A16, e=A4, rs=None, idx=A4, k=2048, swa=A16, ss=None,
             p0=A4, clip=None, W=128, Hq=64, D=1664, sc=0.0245, o8=A16, osc=A4, out=None, lse=None,
             ws=None, nb=0)
    a.update(kw)
    return lib().sparse_mqa_attend_fused(ctypes.byref(L), a["q"], a["rc"], a["rs_"], a["R"], a["c"],
                                         a["e"], a["rs"], a["idx"], a["k"], a["swa"], a["ss"], a["p0"],
                                         a["clip"], a["W"], a["Hq"], a["D"], a["sc"], a["o8"], a["osc"],
                                         a["out"], a["lse"], a["ws"], a["nb"], None)


def test_attend_fused_validation():
    L = layout()
    assert attend_fused(L, R=6) == -4 and "rope_pairs" in err()
    assert attend_fused(L, R=836) == -4 and attend_fused(L, R=-4) == -4
    assert attend_fused(L, rc=None) == -1 and attend_fused(L, rs_=None) == -1
    assert attend_fused(L, R=0, rc=None, rs_=None) == -5          # no rotation: tables optional
    assert attend_fused(L, rc=A16 + 4) == -3
    assert attend_fused(L, o8=None) == -1 and attend_fused(L, osc=None) == -1
    assert attend_fused(L, o8=A16 + 4) == -3 and attend_fused(L, out=A16 + 4) == -3
    assert attend_fused(L, Hq=48) == -4 and attend_fused(L, D=1792) == -4
    need = lib().smqa_attend_fused_workspace_size(ctypes.byref(L), 2048, 128, 64, 1664)
    assert need > 0
    assert attend_fused(L) == -5
    # one split quantises in the attention kernel: the workspace is the plain call's
    for T, kk, W in ((1, 2048, 128), (64, 64, 16), (512, 2048, 128)):
        Lx = layout(T=T, B=T)
        assert (lib().smqa_attend_fused_workspace_size(ctypes.byref(Lx), kk, W, 64, 1664) ==
                lib().smqa_attend_workspace_size(ctypes.byref(Lx), kk, W, 64, 1664))
    assert attend_fused(layout(T=0)) == 0


def test_decode_step_workspace_covers_parts():
    L = layout(max_ctx=524288, T=4, B=4)
    total = lib().smqa_decode_step_workspace_size(ctypes.byref(L), 2048, 0, 128, 64, 1664)
    scores = 4 * 524288 * 4
    tk = lib().smqa_topk_workspace_size(ctypes.byref(L), 2048, 0)
    at = lib().smqa_attend_workspace_size(ctypes.byref(L), 2048, 128, 64, 1664)
    assert total >= scores + 4 * 2048 * 4 + tk + at
    assert lib().smqa_decode_step_workspace_size(None, 2048, 0, 128, 64, 1664) == 0


def test_error_string_cleared_on_success_path():
    assert score(layout(Di=3) if False else layout(), Di=3) == -4
    assert err() != ""
    assert score(layout(T=0)) == 0
    assert err() == ""


def test_attend_plan_fits_the_lds_at_every_supported_shape():
    """Walk the header's limit table (D, Hq, k, W) over query counts that take each kernel
    (few and many (query, head group) pairs) through the host plan: every shape either gets
    a split count whose workgroup fits a CU's 160 KiB of LDS, or is rejected as unsupported
    by the plan query and by every size query and attention call alike."""
    l = lib()
    S = ctypes.c_int32()
    lds = ctypes.c_int32()
    rejected = []
    for D in range(128, 2049, 128):
        for Hq in (16, 32, 48, 64, 96, 128):
            for k in (1, 256, 2048, 4096):
                for W in (1, 128):
                    for T in (1, 4, 64, 1024):
                        L = layout(T=T, B=T)
                        st = l.smqa_attend_plan(ctypes.byref(L), k, W, Hq, D, ctypes.byref(S), ctypes.byref(lds))
                        if st == 0:
                            assert 1 <= S.value <= 64
                            assert 0 < lds.value <= 160 * 1024, (D, Hq, k, W, T, S.value, lds.value)
                            need = l.smqa_attend_workspace_size(ctypes.byref(L), k, W, Hq, D)
                            assert (need == 0) == (S.value == 1)
                        else:
                            assert st == -4 and "LDS" in err()
                            rejected.append((D, Hq, k, W, T))
                            assert l.smqa_attend_workspace_size(ctypes.byref(L), k, W, Hq, D) == 0
                            assert attend(L, k=k, W=W, Hq=Hq, D=D, ws=A16 * 16, nb=1 << 40) == -4
    assert not rejected, rejected[:5]
    # the shapes that overflowed a single-split plan now take more splits
    L = layout(T=64, B=64)
    assert l.smqa_attend_plan(ctypes.byref(L), 2048, 128, 64, 2048, ctypes.byref(S), ctypes.byref(lds)) == 0
    assert S.value > 1 and lds.value <= 160 * 1024
    assert l.smqa_attend_plan(ctypes.byref(L), 2048, 128, 60, 2048, None, None) == -4   # Hq % 16


def decode_noalloc(L, **kw):
    a = dict(qI=A16, w=A4, kI=A16, ks=None, cand=None, n_cand=0, Hi=64, Di=128, q=A16, c=A16, e=A4,
             rs=None, swa=A16, ss=None, p0=A4, clip=None, W=128, Hq=64, D=1664, sc=0.0245, k=2048,
             out=A16, lse=None, idx=None)
    a.update(kw)
    return lib().decode_step_noalloc(ctypes.byref(L), a["qI"], a["w"], a["kI"], a["ks"], a["cand"],
                                     a["n_cand"], a["Hi"], a["Di"], a["q"], a["c"], a["e"], a["rs"],
                                     a["swa"], a["ss"], a["p0"], a["clip"], a["W"], a["Hq"], a["D"],
                                     a["sc"], a["k"], a["out"], a["lse"], a["idx"], None)


def test_decode_step_noalloc_rejects_before_any_hip_call():
    """The no-allocation step validates everything on the host first: bad arguments, and a
    batch whose workspace exceeds the 96 MiB device scratch buffer (a 1024-query replay
    chunk), return an error without a device."""
    cap = 96 << 20
    L = layout(T=1024, B=8, max_ctx=100000)
    need = lib().smqa_decode_step_workspace_size(ctypes.byref(L), 2048, 0, 128, 64, 1664)
    assert need > cap
    assert decode_noalloc(L) == -5 and "scratch" in err()
    assert decode_noalloc(layout(), q=None) == -1
    assert decode_noalloc(layout(), Di=96) == -4
    assert decode_noalloc(layout(), out=A16 + 4) == -3
    assert decode_noalloc(layout(T=0)) == 0
    # the decode batches of the benchmark fit
    for B, T, n in ((1, 1, 8192), (32, 32, 65536), (4, 4, 524288)):
        Lb = layout(T=T, B=B, max_ctx=n)
        assert 0 < lib().smqa_decode_step_workspace_size(ctypes.byref(Lb), 2048, 0, 128, 64, 1664) <= cap


def test_attend_mxfp8q_validation():
    L = layout()

    def call(Lx=L, **kw):
        a = dict(q=A16, c=A16, e=A4, rs=None, idx=A4, k=2048, swa=A16, ss=None, p0=A4, clip=None, W=128,
                 Hq=64, D=1664, sc=0.0245, out=A16, lse=None, ws=None, nb=0)
        a.update(kw)
        return lib().sparse_mqa_attend_mxfp8q(ctypes.byref(Lx), a["q"], a["c"], a["e"], a["rs"], a["idx"],
                                              a["k"], a["swa"], a["ss"], a["p0"], a["clip"], a["W"], a["Hq"],
                                              a["D"], a["sc"], a["out"], a["lse"], a["ws"], a["nb"], None)
    assert call(Hq=48) == -4 and "MXFP8" in err()
    assert call(D=1792) == -4 and call(D=1600) == -4
    assert call(c=None) == -1 and call(e=None) == -1 and call(idx=None) == -1
    assert call(c=A16 + 4) == -3
    assert call() == -5                                      # split partials need the workspace
    assert call(Lx=layout(T=0)) == 0


def test_bench_read_library_rejects_bad_arguments_before_any_hip_call():
    """The benchmark's streaming-read reference (libsmqa_bench.so, built beside the path's
    library) refuses null pointers, sizes that are not whole 16-byte words and unsupported
    depths without touching the device."""
    path = os.path.join(os.path.dirname(smqa.__file__), "libsmqa_bench.so")
    lib = ctypes.CDLL(path)
    fn = lib.smqa_bench_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_void_p]
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    assert fn(None, 1 << 20, p, 256, 4, None) == -1
    assert fn(p, 1 << 20, None, 256, 4, None) == -1
    assert fn(p, 17, p, 256, 4, None) == -1
    assert fn(p, 0, p, 256, 4, None) == -1
    assert fn(p, 1 << 20, p, 0, 4, None) == -1
    assert fn(p, 1 << 20, p, 256, 3, None) == -1


def test_debug_flags_outside_a_debug_build_and_in_one():
    """smqa_debug_flags: SMQA_ERR_NULL for a null pointer in either build; the release
    library answers SMQA_ERR_UNSUPPORTED with the word zeroed, without touching a device.
    The debug library (same sources, SMQA_DEBUG) exports every symbol the header declares."""
    rel = smqa.load()
    v = ctypes.c_uint32(7)
    assert rel.smqa_debug_flags(None, 1) == -1
    assert rel.smqa_debug_flags(ctypes.byref(v), 1) == -4
    assert v.value == 0
    assert b"not an SMQA_DEBUG build" in rel.smqa_last_error()
    with pytest.raises(smqa.SmqaError):
        smqa.debug_flags()
    dbg = ctypes.CDLL(smqa.DEBUG_LIB_PATH)
    for name in declared_functions():
        assert hasattr(dbg, name), name
    assert dbg.smqa_debug_flags(None, 1) == -1


def score_fp8mma(L, Hi=64, Di=128, **kw):
    a = dict(q=A16, w=A4, k=A16, ks=None, cand=None, n_cand=0, s=A4, ld=8192)
    a.update(kw)
    if L is None:
        return lib().sparse_mqa_score_fp8mma(None, a["q"], a["w"], a["k"], a["ks"], a["cand"], a["n_cand"],
                                             Hi, Di, a["s"], a["ld"], None)
    return lib().sparse_mqa_score_fp8mma(ctypes.byref(L), a["q"], a["w"], a["k"], a["ks"], a["cand"],
                                         a["n_cand"], Hi, Di, a["s"], a["ld"], None)


def test_score_fp8mma_validation():
    """The FP8 matrix-core form validates like sparse_mqa_score and also rejects Di != 128,
    all before any HIP call."""
    L = layout()
    assert score_fp8mma(None) == -1
    assert score_fp8mma(L, q=None) == -1 and "q_fp8" in err()
    assert score_fp8mma(L, Di=96) == -4
    assert score_fp8mma(L, Di=64) == -4 and "Di = 128" in err()
    assert score_fp8mma(L, ld=100) == -2
    assert score_fp8mma(layout(T=0)) == 0
