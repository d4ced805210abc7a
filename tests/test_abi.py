"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/w4a8.h declares, and rejects bad arguments on the host before
any HIP call (pointers below are fake addresses that are never dereferenced).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")

w4 = pytest.importorskip("w4a8_quantized_gemm_amd")
lib = w4.lib

OK, NULL, SHAPE, ALIGN, WS, UNSUP, HIP = range(7)
A = 0x10000  # a 16-byte-aligned fake device address, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return set(re.findall(r"^\s*(?:w4a8_status_t|size_t|int|const char\*)\s+(\w+)\s*\(",
                          text, re.M))


def test_exports_match_header():
    names = declared_functions()
    assert names == set(w4.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_layout_version_and_strings():
    assert lib.w4a8_layout_version() == 1
    for s in range(7):
        assert lib.w4a8_status_str(s)
    assert lib.w4a8_status_str(99) == b"unknown status"
    assert lib.w4a8_workspace_size(16, 4096, 4096, 0) == 0


def pack(W=A, N=64, K=256, g=64, qmax=127, mode=0, wq=A, s=A, a=A, sw=A):
    return lib.w4a8_pack(W, N, K, g, qmax, mode, wq, s, a, sw, None)


def test_pack_validation():
    assert pack(W=None) == NULL
    assert pack(wq=None) == NULL
    assert pack(s=None) == NULL
    assert pack(mode=1, s=None, a=None, g=0, qmax=0) != NULL  # INT4: s/a unused
    assert pack(N=0, W=None, wq=None) == OK  # empty: pointers not read
    assert pack(mode=7) == UNSUP
    assert pack(K=200) == SHAPE
    assert pack(K=0) == SHAPE
    assert pack(N=24) == SHAPE
    assert pack(N=-16) == SHAPE
    assert pack(g=32) == SHAPE
    assert pack(qmax=0) == SHAPE
    assert pack(qmax=128) == SHAPE
    assert pack(W=A + 4) == ALIGN
    assert pack(wq=A + 8) == ALIGN
    assert pack(N=0) == OK  # empty problem, nothing launched


def gemm(X=A, sx=A, wq=A, s=A, a=A, sw=A, Y=A, out=0, M=16, N=64, K=256, g=64,
         splitk=0, ws=None, wsb=0):
    return lib.w4a8_gemm(X, sx, wq, s, a, sw, Y, out, M, N, K, g, splitk, ws, wsb, None)


def test_gemm_validation():
    assert gemm(X=None) == NULL
    assert gemm(Y=None) == NULL
    assert gemm(sx=None) == NULL
    assert gemm(sx=None, sw=None, out=1, M=0) == OK  # int32 output needs no scales
    assert gemm(out=5) == UNSUP
    assert gemm(M=-1) == SHAPE
    assert gemm(K=192) == SHAPE
    assert gemm(N=40) == SHAPE
    assert gemm(N=48) == SHAPE  # N must be a multiple of 64
    assert gemm(g=256) == SHAPE
    assert gemm(splitk=3) == SHAPE
    assert gemm(splitk=4, K=256) == SHAPE  # more slices than K tiles
    assert gemm(splitk=32, K=8192) == SHAPE
    assert gemm(X=A + 1) == ALIGN
    assert gemm(Y=A + 2) == ALIGN
    assert gemm(sx=A + 2) == ALIGN
    assert gemm(M=0) == OK
    assert gemm(N=0) == OK
    assert gemm(M=0, X=None, Y=None) == OK  # empty: pointers not read
    assert gemm(M=0, K=100) == SHAPE


def fp8(X=A, sx=A, wq=A, sw=A, Y=A, out=0, M=16, N=64, K=256, splitk=0):
    return lib.w4fp8_gemm(X, sx, wq, sw, Y, out, M, N, K, splitk, None, 0, None)


def test_fp8_gemm_validation():
    assert fp8(X=None) == NULL
    assert fp8(sw=None) == NULL
    assert fp8(out=2) == UNSUP
    assert fp8(K=100) == SHAPE
    assert fp8(N=8) == SHAPE
    assert fp8(wq=A + 4) == ALIGN
    assert fp8(M=0) == OK


def test_quant_act_validation():
    f = lib.w4a8_quant_act
    g = lib.w4fp8_quant_act
    for fn in (f, g):
        assert fn(None, 4, 64, A, A, None) == NULL
        assert fn(A, 4, 60, A, A, None) == SHAPE
        assert fn(A, -1, 64, A, A, None) == SHAPE
        assert fn(A + 4, 4, 64, A, A, None) == ALIGN
        assert fn(A, 0, 64, A, A, None) == OK


def test_gemm_ablation_validation():
    def abl(variant=1, M=256, N=256, K=512, g=128, out=0, X=A, wq=A, s=A, a=A, Y=A):
        return lib.w4a8_gemm_ablation(variant, X, A, wq, s, a, A, Y, out, M, N, K, g, None)
    assert abl(variant=3) == UNSUP
    assert abl(variant=-1) == UNSUP
    assert abl(out=2) == UNSUP
    assert abl(K=100) == SHAPE
    assert abl(g=32) == SHAPE
    assert abl(M=0) == OK
    for v in (0, 1, 2):
        assert abl(variant=v, M=16) == UNSUP          # streamed-kernel shape
        assert abl(variant=v, N=192) == UNSUP         # N % 256 != 0
        assert abl(variant=v, M=128, K=8192) == UNSUP  # the plan splits K
        assert abl(variant=v, wq=None) == NULL
        assert abl(variant=v, X=A + 4) == ALIGN


def test_gemm_grouped_validation():
    def grp(M=64, E=4, N=256, K=512, g=64, out=0, rows=16, X=A, off=A, wq=A, Y=A):
        return lib.w4a8_gemm_grouped(X, A, off, E, wq, A, A, A, Y, out, M, N, K, g, rows, None)
    assert grp(out=2) == UNSUP
    assert grp(E=0) == SHAPE
    assert grp(K=100) == SHAPE
    assert grp(N=48) == SHAPE
    assert grp(g=32) == SHAPE
    assert grp(rows=-1) == SHAPE
    assert grp(M=1 << 20, K=4096) == SHAPE      # M*K >= 2^31
    assert grp(M=0) == OK
    assert grp(rows=0) == OK
    assert grp(off=None) == NULL
    assert grp(wq=None) == NULL
    assert grp(off=A + 2) == ALIGN
    assert grp(X=A + 4) == ALIGN


def test_quant_act_ex_validation():
    for fn in (lib.w4a8_quant_act_ex, lib.w4fp8_quant_act_ex):
        for it in (0, 1, 2):
            assert fn(None, it, 4, 64, A, A, None) == NULL
            assert fn(A, it, 4, 60, A, A, None) == SHAPE
            assert fn(A, it, -1, 64, A, A, None) == SHAPE
            assert fn(A + 8, it, 4, 64, A, A, None) == ALIGN
            assert fn(A, it, 4, 64, A + 8, A, None) == ALIGN
            assert fn(A, it, 0, 64, A, A, None) == OK
        assert fn(A, 3, 4, 64, A, A, None) == UNSUP
        assert fn(A, -1, 4, 64, A, A, None) == UNSUP


def test_fp8_group_fold_validation():
    def gp(W=A, N=64, K=256, g=128, wq=A, f=A, t=A):
        return lib.w4fp8g_pack(W, N, K, g, wq, f, t, None)
    assert gp(g=32) == SHAPE
    assert gp(K=100) == SHAPE
    assert gp(N=8) == SHAPE
    assert gp(N=0) == OK
    assert gp(f=None) == NULL
    assert gp(t=None) == NULL
    assert gp(W=A + 4) == ALIGN
    assert gp(t=A + 2) == ALIGN

    def gg(M=16, N=256, K=512, g=64, out=0, splitk=0, X=A, f=A, t=A, Y=A, ws=0, wsb=0):
        return lib.w4fp8g_gemm(X, A, A, f, t, Y, out, M, N, K, g, splitk, ws, wsb, None)
    assert gg(out=2) == UNSUP
    assert gg(g=96) == SHAPE
    assert gg(K=100) == SHAPE
    assert gg(splitk=3) == SHAPE
    assert gg(M=0) == OK
    assert gg(f=None) == NULL
    assert gg(t=None) == NULL
    assert gg(Y=A + 4) == ALIGN
    need = lib.w4a8_workspace_size(128, 256, 8192, 0)
    assert need > 0
    assert gg(M=128, K=8192, wsb=need - 1, ws=A) == WS
    assert gg(M=128, K=8192, wsb=need, ws=0) == NULL


def test_w8a8_validation():
    def pk(W=A, N=64, K=256, wq=A, sw=A):
        return lib.w8a8_pack(W, N, K, wq, sw, None)
    assert pk(K=100) == SHAPE
    assert pk(N=8) == SHAPE
    assert pk(N=1 << 16, K=1 << 15) == SHAPE   # N*K >= 2^31
    assert pk(N=0) == OK
    assert pk(wq=None) == NULL
    assert pk(W=A + 4) == ALIGN

    def gm(M=16, N=256, K=512, out=0, splitk=0, X=A, wq=A, sx=A, sw=A, Y=A, ws=0, wsb=0):
        return lib.w8a8_gemm(X, sx, wq, sw, Y, out, M, N, K, splitk, ws, wsb, None)
    assert gm(out=2) == UNSUP
    assert gm(K=100) == SHAPE
    assert gm(splitk=3) == SHAPE
    assert gm(M=0) == OK
    assert gm(wq=None) == NULL
    assert gm(sw=None) == NULL
    assert gm(Y=A + 4) == ALIGN
    need = lib.w4a8_workspace_size(128, 256, 8192, 0)
    assert gm(M=128, K=8192, ws=A, wsb=need - 1) == WS


def test_gemm_extent_limits():
    """M*K >= 2^31 or N*K >= 2^32 is rejected before any HIP call, by every
    GEMM entry point (sizes only; the fake pointers are never used)."""
    big_m, k = 1 << 20, 4096            # M*K = 2^32
    n_big = 1 << 20                     # N*K = 2^32 at K = 4096
    assert lib.w4a8_gemm(A, A, A, A, A, A, A, 0, big_m, 256, k, 128, 0, None, 0, None) == SHAPE
    assert lib.w4a8_gemm(A, A, A, A, A, A, A, 0, 16, n_big, k, 128, 0, None, 0, None) == SHAPE
    assert lib.w4fp8_gemm(A, A, A, A, A, 0, big_m, 256, k, 0, None, 0, None) == SHAPE
    assert lib.w4fp8_gemm(A, A, A, A, A, 0, 16, n_big, k, 0, None, 0, None) == SHAPE
    assert lib.w8a8_gemm(A, A, A, A, A, 0, big_m, 256, k, 0, None, 0, None) == SHAPE
    assert lib.w4a8_gemm_ablation(1, A, A, A, A, A, A, A, 0, big_m, 256, k, 128, None) == SHAPE
    assert lib.w4a8_gemm_grouped(A, A, A, 2, A, A, A, A, A, 0, 16, n_big, k, 128, 8,
                                 None) == SHAPE
    assert lib.w4fp8g_gemm(A, A, A, A, A, A, 0, big_m, 256, k, 128, 0, None, 0, None) == SHAPE
    # just inside the limits the sizes are accepted (validation then stops at
    # the NULL output pointer, before any HIP call)
    assert lib.w4a8_gemm(A, A, A, A, A, A, None, 0, (1 << 19) - 1, 256, k, 128, 0, None, 0,
                         None) == NULL


def test_valid_call_without_gpu_reports_hip_error():
    """A call that passes validation reaches the HIP runtime; with no GPU
    the device query fails and the status is W4A8_ERR_HIP, not a crash."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    st = gemm()
    assert st in (HIP, UNSUP)
    if st == HIP:
        assert lib.w4a8_last_hip_error() != 0


def test_alignment_rule():
    """Byte arrays (including the group parameters, which the streamed
    kernel copies in 16-byte pieces) need 16-byte alignment; the float32 /
    int32 vectors need 4.  A misaligned pointer is rejected before any HIP
    call; a 4-byte-aligned scale vector passes the alignment check."""
    assert gemm(s=A + 4) == ALIGN
    assert gemm(a=A + 8) == ALIGN
    assert gemm(sw=A + 2) == ALIGN
    assert gemm(sw=A + 4) != ALIGN and gemm(sx=A + 4) != ALIGN
    assert pack(s=A + 4) == ALIGN
    assert pack(a=A + 2) == ALIGN
    assert pack(mode=1, s=A + 4, a=A + 2, g=0, qmax=0) != ALIGN  # INT4: s/a unused
    assert lib.w4a8_gemm_ablation(0, A, A, A, A + 4, A, A, A, 0, 256, 256, 512, 128,
                                  None) == ALIGN
    assert lib.w4a8_gemm_grouped(A, A, A, 4, A, A, A + 8, A, A, 0, 64, 256, 512, 64, 16,
                                 None) == ALIGN
    assert lib.w4a8_gemm_grouped(A, A, A + 4, 4, A, A, A, A, A, 0, 64, 256, 512, 64, 16,
                                 None) != ALIGN


def test_binding_checks_sizes_before_any_launch():
    """The Python binding compares every operand's size with the call's
    M, N, K (and group) before a pointer reaches the library, so a wrongly
    sized output, scale vector or packed array cannot be read or written
    past its end.  CPU tensors of the right sizes get past these checks and
    stop at the device check, so nothing here launches anything."""
    torch = pytest.importorskip("torch")
    M, N, K, g = 16, 256, 512, 64
    X = torch.zeros((M, K), dtype=torch.int8)
    sx = torch.ones(M)
    pk = {"wq": torch.zeros(N * K // 2, dtype=torch.uint8),
          "s_u8": torch.ones(N * K // g, dtype=torch.uint8),
          "a_u8": torch.ones(N * K // g, dtype=torch.uint8),
          "sw": torch.ones(N), "N": N, "K": K, "group": g}
    for fn in (w4.gemm, lambda *a, **k: w4.gemm_ablation(w4.ABL_LQQ, *a, **k)):
        with pytest.raises(ValueError, match="out"):
            fn(X, sx, pk, out=torch.empty((M, N - 64), dtype=torch.float16))
        with pytest.raises(ValueError, match="sx"):
            fn(X, sx[:M - 1], pk)
        for key in ("wq", "s_u8", "a_u8", "sw"):
            with pytest.raises(ValueError, match=key):
                fn(X, sx, dict(pk, **{key: pk[key][:-16]}))
        with pytest.raises(ValueError, match="GPU"):
            fn(X, sx, pk)
    with pytest.raises(ValueError, match="K of X"):
        w4.gemm(torch.zeros((M, K + 128), dtype=torch.int8), sx, pk)
    # grouped: E experts' arrays end to end
    E = 2
    pke = {k: (torch.cat([v, v]) if torch.is_tensor(v) else v) for k, v in pk.items()}
    pke["E"] = E
    offs = torch.tensor([0, 8, M], dtype=torch.int32)
    with pytest.raises(ValueError, match="out"):
        w4.gemm_grouped(X, sx, offs, pke, 8, out=torch.empty((M + 1, N), dtype=torch.float16))
    with pytest.raises(ValueError, match="wq"):
        w4.gemm_grouped(X, sx, offs, dict(pke, wq=pk["wq"]), 8)
    with pytest.raises(ValueError, match="GPU"):
        w4.gemm_grouped(X, sx, offs, pke, 8)
    # FP8 per-channel and folded, W8A8
    Xe = torch.zeros((M, K), dtype=torch.uint8)
    pf = {"wq": pk["wq"], "sw": pk["sw"], "N": N, "K": K}
    with pytest.raises(ValueError, match="out"):
        w4.gemm_fp8(Xe, sx, pf, out=torch.empty((M, N), dtype=torch.bfloat16)[:, :128])
    with pytest.raises(ValueError, match="sw"):
        w4.gemm_fp8(Xe, sx, dict(pf, sw=pk["sw"][:-1]))
    pg = {"wq": pk["wq"], "fsc": torch.ones((K // g, N)), "tscale": torch.ones(1),
          "N": N, "K": K, "group": g}
    with pytest.raises(ValueError, match="fsc"):
        w4.gemm_fp8g(Xe, sx, dict(pg, fsc=torch.ones((K // g, N - 64))))
    with pytest.raises(ValueError, match="GPU"):
        w4.gemm_fp8g(Xe, sx, pg)
    p8 = {"wq8": torch.zeros(N * K, dtype=torch.int8), "sw": pk["sw"], "N": N, "K": K}
    with pytest.raises(ValueError, match="wq8"):
        w4.gemm_w8a8(X, sx, dict(p8, wq8=pk["wq"]))
    with pytest.raises(ValueError, match="sx"):
        w4.gemm_w8a8(X, torch.ones(M + 3), p8)


def test_gemm_noalloc_validation():
    """w4a8_gemm_noalloc validates exactly as w4a8_gemm does, before any HIP
    call (no workspace argument: the library's static scratch stands in)."""
    def na(X=A, sx=A, wq=A, s=A, a=A, sw=A, Y=A, out=0, M=16, N=64, K=256, g=64, splitk=0):
        return lib.w4a8_gemm_noalloc(X, sx, wq, s, a, sw, Y, out, M, N, K, g, splitk, None)
    assert na(X=None) == NULL
    assert na(sx=None) == NULL
    assert na(out=5) == UNSUP
    assert na(K=192) == SHAPE
    assert na(splitk=3) == SHAPE
    assert na(s=A + 4) == ALIGN
    assert na(M=0, X=None, Y=None) == OK
    # a split-K shape: needs partials, none are passed, still not a NULL error
    assert lib.w4a8_workspace_size(128, 512, 8192, 0) > 0
    assert na(M=128, N=512, K=8192) in (HIP, UNSUP)
