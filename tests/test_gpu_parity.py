"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Bars: bit-exact for packed bytes, codes, scales and int32 accumulators;
fp16 output within 1 ulp of the oracle's once-rounded double result; FP8
variant within relative Frobenius error 1e-3 of the double reference (the
float32 output), and of the bfloat16-rounded double reference (the bfloat16
output).  Small cases run against the full oracle; the Llama-shaped
workloads run in the launch configuration the benchmark uses and are
checked on sampled rows and columns (the oracle quantises per row, so a row
sample is computed exactly as in the full problem).
"""
import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a8_quantized_gemm_amd as w4  # noqa: E402  (must load: no fallback)

DEV = "cuda:0"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def poison(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(0xAB)
    return t


def f16_ulp_diff(a_bits, b_bits):
    def ordered(u):
        u = u.astype(np.int64)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def bf16_bits_of(t):
    return host(t.view(torch.int16)).view(np.uint16)


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------ packing ------
@pytest.mark.parametrize("N,K,g,qmax", [(256, 512, 64, 127), (64, 384, 64, 119),
                                        (64, 1024, 128, 127), (4096, 4096, 64, 127)])
def test_pack_lqq_parity(N, K, g, qmax):
    say(f"pack lqq N={N} K={K} g={g} qmax={qmax}")
    W = wl.gen_weights(N, K, 100 + N)
    W[3] = 0.0  # all-zero channel
    ref = oracle.w4a8_pack(W, g, qmax)
    pk = w4.pack(to_dev(W), group=g, qmax=qmax)
    np.testing.assert_array_equal(host(pk["sw"]), ref["sw"])
    np.testing.assert_array_equal(host(pk["s_u8"]), ref["s_panels"])
    np.testing.assert_array_equal(host(pk["a_u8"]), ref["a_panels"])
    np.testing.assert_array_equal(host(pk["wq"]), ref["wq"])


@pytest.mark.parametrize("N,K", [(256, 512), (192, 1024)])
def test_pack_int4_parity(N, K):
    say(f"pack int4 N={N} K={K}")
    W = wl.gen_weights(N, K, 200 + N)
    ref = oracle.w4fp8_pack(W)
    pk = w4.pack(to_dev(W), mode=w4.PACK_INT4_SYM)
    np.testing.assert_array_equal(host(pk["sw"]), ref["sw"])
    np.testing.assert_array_equal(host(pk["wq"]), ref["wq"])


# ------------------------------------------------- activation quant --------
# Rows of up to 32768 elements are held in registers: with fewer than 256
# rows 1024 threads per row hold 1, 2 or 4 pieces of eight each (K up to
# 8192, 16384, 28672), from 256 rows on 256 threads hold 2, 4, 8 or 16
# (K = 2048, 8192, 16384, 28672); longer rows (33024) take the two-pass
# kernels.
@pytest.mark.parametrize("M,K", [(1, 512), (16, 4096), (33, 1024), (3, 8192), (5, 16384),
                                 (2, 28672), (3, 33024), (300, 2048), (256, 8192),
                                 (257, 16384), (256, 28672), (256, 33024)])
def test_quant_act_parity(M, K):
    say(f"quant act M={M} K={K}")
    X = wl.gen_activations(M, K, 300 + M, 301)
    if M > 2:
        X[1] = 0.0
    q8, s8 = oracle.quant_sym_rows(X, 127)
    Xq, sx = w4.quant_act(to_dev(X))
    np.testing.assert_array_equal(host(sx), s8)
    np.testing.assert_array_equal(host(Xq), q8)
    qf, sf = oracle.quant_rows_e4m3(X)
    Xf, sxf = w4.quant_act_fp8(to_dev(X))
    np.testing.assert_array_equal(host(sxf), sf)
    np.testing.assert_array_equal(host(Xf), qf)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("M,K", [(1, 512), (16, 4096), (37, 1040), (4, 8192), (4, 28672),
                                 (4, 33024), (260, 4096), (256, 28672)])
def test_quant_act_typed_parity(dt, M, K):
    """fp16 / bf16 activations: the device widens to float32 and quantises;
    the oracle widens the same bit patterns (exact) and quantises.  Rows:
    Gaussian with outlier channels, an all-zero row, a row of the format's
    smallest subnormals and signed zeros, and a row at the largest finite
    value."""
    say(f"quant act {dt} M={M} K={K}")
    X = wl.gen_activations(M, K, 310 + M, 311).astype(np.float64)
    if dt == "f16":
        bits = oracle.round_f16(X)
        tiny, big = 0x0001, 0x7BFF
        widen, tdt = oracle.widen_f16, torch.float16
    else:
        bits = oracle.round_bf16(X)
        tiny, big = 0x0001, 0x7F7F
        widen, tdt = oracle.widen_bf16, torch.bfloat16
    if M > 3:
        bits[1] = 0
        bits[2] = np.where(np.arange(K) % 2 == 0, tiny, 0x8000 | tiny)
        bits[2, ::3] = 0x8000
        bits[3] = np.where(np.arange(K) % 5 == 0, 0x8000 | big, bits[3])
    Xw = widen(bits)
    Xd = to_dev(bits.view(np.int16)).view(tdt)
    q8, s8 = oracle.quant_sym_rows(Xw, 127)
    Xq, sx = w4.quant_act(Xd)
    np.testing.assert_array_equal(host(sx), s8)
    np.testing.assert_array_equal(host(Xq), q8)
    qf, sf = oracle.quant_rows_e4m3(Xw)
    Xf, sxf = w4.quant_act_fp8(Xd)
    np.testing.assert_array_equal(host(sxf), sf)
    np.testing.assert_array_equal(host(Xf), qf)


# ------------------------------------------------------- W4A8 GEMM ---------
def _small_problem(M, N, K, g, seed):
    W = wl.gen_weights(N, K, seed)
    X = wl.gen_activations(M, K, seed + 1, seed + 2)
    pk_ref = oracle.w4a8_pack(W, g)
    X8, sx = oracle.quant_sym_rows(X, 127)
    acc, y, _ = oracle.w4a8_gemm(X8, sx, pk_ref, g)
    pk = {"wq": to_dev(pk_ref["wq"]), "s_u8": to_dev(pk_ref["s_panels"]),
          "a_u8": to_dev(pk_ref["a_panels"]), "sw": to_dev(pk_ref["sw"]),
          "N": N, "K": K, "group": g}
    return to_dev(X8), to_dev(sx), pk, acc, y


@pytest.mark.parametrize("M", list(range(1, 18)) + [33, 100])
@pytest.mark.parametrize("N,K,g", [(128, 640, 64), (64, 512, 128), (128, 128, 64)])
def test_w4a8_gemm_parity(M, N, K, g):
    say(f"w4a8 gemm M={M} N={N} K={K} g={g}")
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 1000 + M)
    Yi = poison((M, N), torch.int32)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi)
    np.testing.assert_array_equal(host(Yi), acc)
    Yh = poison((M, N), torch.float16)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh)
    d = f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y)
    assert d.max() <= 1


# Degenerate inputs of the method through the GEMM kernels: channels whose
# groups have zero range (all zero, constant: s = 1, q = 0, decode = min),
# alternate +-max|w| (every group spans the full INT8 range: the saturation
# branch), a narrow range (R <= 15: lossless), one outlier per group, and the
# largest and smallest per-channel scales side by side; activation rows all
# zero (scale 1, codes 0), at +-qmax everywhere, and alternating signs.
@pytest.mark.parametrize("M", [7, 100])
@pytest.mark.parametrize("g", [64, 128])
def test_degenerate_weights_and_rows(M, g):
    N, K = 256, 1024
    say(f"degenerate weights and rows M={M} g={g}")
    W = wl.gen_weights(N, K, 5100 + g)
    W[0] = 0.0
    W[1] = 0.5
    W[2] = np.where(np.arange(K) % 2 == 0, 1.0, -1.0)
    W[3] = 0.01 + 1e-4 * (np.arange(K) % 7)
    W[4, ::g] = 3.0
    W[5] *= 1e-30
    W[6] *= 1e6
    X = wl.gen_activations(M, K, 5200 + M, 5201)
    X[0] = 0.0
    X[1] = 2.0
    X[2] = np.where(np.arange(K) % 3 == 0, -1.5, 1.5)
    X[3, :g] = 0.0
    pk_ref = oracle.w4a8_pack(W, g)
    X8, sx = oracle.quant_sym_rows(X, 127)
    acc, y, _ = oracle.w4a8_gemm(X8, sx, pk_ref, g)
    pk = {"wq": to_dev(pk_ref["wq"]), "s_u8": to_dev(pk_ref["s_panels"]),
          "a_u8": to_dev(pk_ref["a_panels"]), "sw": to_dev(pk_ref["sw"]),
          "N": N, "K": K, "group": g}
    for sk in (0, 1):
        Yi = poison((M, N), torch.int32)
        w4.gemm(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_I32, splitk=sk, out=Yi)
        np.testing.assert_array_equal(host(Yi), acc)
        Yh = poison((M, N), torch.float16)
        w4.gemm(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F16, splitk=sk, out=Yh)
        d = f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y)
        assert d.max() <= 1
    # the device pack of the same weights gives the same codes
    dpk = w4.pack(to_dev(W), group=g)
    np.testing.assert_array_equal(host(dpk["wq"]), pk_ref["wq"])
    np.testing.assert_array_equal(host(dpk["s_u8"]), pk_ref["s_panels"])
    np.testing.assert_array_equal(host(dpk["a_u8"]), pk_ref["a_panels"])


# Shapes that the dispatcher sends to the matrix-core tile kernels (N a
# multiple of 256, M >= 64): 128-row tiles (short K: two per CU on the
# 16 x 16 x 64 kernel), ragged M, and odd
# K-step counts (640 = 5 steps, 896 = 7): an odd count runs one extra step of
# zero X, and the accumulators' last writes must be complete before the
# epilogue reads them.  K = 128 is a single K-step (the loop's second step is
# all zero X).
@pytest.mark.parametrize("M", [64, 65, 100, 128, 129, 200, 256, 257, 300, 513, 777])
@pytest.mark.parametrize("N,K,g", [(256, 512, 64), (512, 1024, 128), (1024, 640, 128),
                                   (512, 896, 64), (256, 128, 64), (512, 128, 128)])
def test_w4a8_gemm_mfma_parity(M, N, K, g):
    say(f"w4a8 mfma gemm M={M} N={N} K={K} g={g}")
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 2000 + M)
    Yi = poison((M, N), torch.int32)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi)
    np.testing.assert_array_equal(host(Yi), acc)
    Yh = poison((M, N), torch.float16)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh)
    d = f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y)
    assert d.max() <= 1
    # the streamed-tile kernel (forced by an explicit split) agrees
    Ys = poison((M, N), torch.int32)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, splitk=2 if K >= 256 else 1, out=Ys)
    np.testing.assert_array_equal(host(Ys), acc)


def test_mfma_tiles_full_grid():
    """A grid large enough for the XCD regrouping (workgroup count a
    multiple of 8)."""
    M, N, K, g = 1024, 2048, 512, 64
    say(f"w4a8 mfma gemm M={M} N={N} K={K} g={g}")
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 31)
    Yi = poison((M, N), torch.int32)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi)
    np.testing.assert_array_equal(host(Yi), acc)


# Large grids (at least 256 tiles of 256 rows: M x N = 4096 x 4096 and more)
# with short K, which run 128-row tiles two per CU (256-row tiles, kept for
# long K, are covered by test_256_row_tiles_long_k).  K = 384 gives an odd
# number of K-steps (the unrolled loop's tail step).
@pytest.mark.parametrize("M,N,K,g", [(4000, 4096, 384, 128), (4096, 4096, 512, 64)])
def test_large_grid_tiles(M, N, K, g):
    say(f"w4a8 large-grid gemm M={M} N={N} K={K} g={g}")
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 41 + K)
    Yi = poison((M, N), torch.int32)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi)
    np.testing.assert_array_equal(host(Yi), acc)
    Yh = poison((M, N), torch.float16)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh)
    d = f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y)
    assert d.max() <= 1


# Several waves of tiles (512, 544 and 768 tiles of 256 rows, run as 128-row
# tiles two per CU): ragged M, K-step counts 2 and 4, a partial last wave.
@pytest.mark.parametrize("M,N,K,g", [(4000, 8192, 512, 128), (4352, 8192, 256, 64),
                                     (4096, 12288, 512, 64)])
def test_large_grid_several_waves(M, N, K, g):
    say(f"w4a8 gemm, several waves of tiles: M={M} N={N} K={K} g={g}")
    assert w4.workspace_size(M, N, K) == 0
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 61 + K)
    Yi = poison((M, N), torch.int32)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi)
    np.testing.assert_array_equal(host(Yi), acc)
    Yh = poison((M, N), torch.float16)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh)
    d = f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y)
    assert d.max() <= 1


# Every configuration of the streamed kernel (M < 64): one 16-row block per
# workgroup with 4, 2 and 1 tiles (N = 10240 / 14336, 8192, 4096); two
# blocks per workgroup with 4, 2 and 1 tiles (at 48 and 50 rows the second
# workgroup along M holds one block partly and one wholly past M); four
# blocks (33-63 rows) with 2 tiles.  Short K leaves
# waves with fewer K-tiles than the load ring holds (640 / 128 = 5 K-tiles
# over 4 waves, 1152 over 8 waves).  The last case holds too many group
# parameters for LDS (512 groups per channel row: parameter panels plus X
# slots past 128 KiB), so each tile reads its scale and offset bytes from
# memory with one row block and 128-wide groups (test_stream_params_from_global
# covers two row blocks and 64-wide groups).
@pytest.mark.parametrize("M,N,K,g", [(16, 10240, 1024, 128), (1, 14336, 640, 64),
                                     (16, 8192, 2048, 128), (7, 4096, 512, 64),
                                     (32, 28672, 640, 128), (20, 8192, 1024, 64),
                                     (17, 4096, 768, 128), (48, 4096, 768, 64),
                                     (33, 8192, 1152, 64), (40, 28672, 512, 128),
                                     (63, 11008, 512, 64), (50, 2048, 2048, 64),
                                     (20, 2048, 65536, 128)])
def test_stream_widths(M, N, K, g):
    say(f"w4a8 streamed kernel widths: M={M} N={N} K={K} g={g}")
    assert w4.workspace_size(M, N, K) == 0
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 81 + M)
    Yi = poison((M, N), torch.int32)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi)
    np.testing.assert_array_equal(host(Yi), acc)
    Yh = poison((M, N), torch.float16)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh)
    d = f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y)
    assert d.max() <= 1


# Few output tiles -> the matrix-core kernel splits K across workgroups and
# reduces int32 partials in a second kernel (128 x 512 x 4096: two splits of
# two K parts each; 100 x 256 x 2048: one workgroup per 128 channels, two K
# parts, no partials).
@pytest.mark.parametrize("M,N,K,g", [(128, 512, 4096, 128), (100, 256, 2048, 64)])
def test_mfma_split_k(M, N, K, g):
    say(f"w4a8 mfma split-K gemm M={M} N={N} K={K} g={g} ws={w4.workspace_size(M, N, K)}")
    assert w4.workspace_size(M, N, K) > 0
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 51 + M)
    Yi = poison((M, N), torch.int32)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi)
    np.testing.assert_array_equal(host(Yi), acc)
    Yh = poison((M, N), torch.float16)
    # a poisoned workspace (scratch: its contents on entry are ignored), then
    # the same workspace again
    ws = poison((w4.workspace_size(M, N, K),), torch.uint8)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh, workspace=ws)
    d = f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y)
    assert d.max() <= 1
    Yh = poison((M, N), torch.float16)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh, workspace=ws)
    d = f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y)
    assert d.max() <= 1


@pytest.mark.parametrize("M,N,K,g", [(256, 512, 512, 128), (300, 256, 768, 64),
                                     (100, 512, 512, 64), (512, 1024, 896, 128),
                                     (256, 1024, 640, 64), (2048, 8192, 512, 64)])
def test_ablation_variants_bit_identical(M, N, K, g):
    """The conventional affine decode and the coarse pipeline produce the
    same int32 accumulators (bit-exact vs the oracle) and the same fp16 as
    the production kernel.  Shapes the unsplit tile kernels serve: 128-row
    tiles with one to seven K-steps, and a grid of 256 tiles of 256 rows
    (last case: the ablation kernels run 256-row tiles there, the product
    path 128-row tiles two per CU)."""
    say(f"ablation variants M={M} N={N} K={K} g={g}")
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 11)
    ref16 = None
    for v in (w4.ABL_LQQ, w4.ABL_AFFINE16, w4.ABL_LQQ_COARSE):
        Yi = poison((M, N), torch.int32)
        w4.gemm_ablation(v, X8, sx, pk, out_type=w4.OUT_I32, out=Yi)
        np.testing.assert_array_equal(host(Yi), acc)
        Yh = poison((M, N), torch.float16)
        w4.gemm_ablation(v, X8, sx, pk, out_type=w4.OUT_F16, out=Yh)
        bits = host(Yh.view(torch.int16))
        if ref16 is None:
            ref16 = bits
            assert f16_ulp_diff(bits.view(np.uint16), y).max() <= 1
        np.testing.assert_array_equal(bits, ref16)


@pytest.mark.parametrize("counts,N,K,g", [
    ([5, 0, 16, 19], 256, 512, 64),          # streamed kernel; an empty expert
    ([1, 1, 1, 1, 1, 1, 1, 1], 512, 640, 128),  # one row each (decode, top-1)
    ([33, 7, 0, 40], 128, 1024, 64),          # ragged, several 16-row blocks
    ([20, 3, 17, 0, 9, 31, 2, 18], 1280, 512, 128),  # streamed, 4 tiles, two row blocks
    ([70, 0, 130, 300], 512, 640, 128),       # matrix-core tiles, odd K-steps
    ([257, 64, 1], 256, 512, 64),             # tiles; an expert with one row
    ([1100, 0, 37, 1500], 256, 512, 128),     # >= 1024 rows: two tile workgroups per CU
])
def test_grouped_gemm_parity(counts, N, K, g):
    """Each expert's rows equal w4a8_gemm of those rows against that
    expert's weights: int32 bit-exact, fp16 within 1 ulp; rows past every
    expert's range are not written."""
    E = len(counts)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offs[-1]) + 3                  # three trailing rows no expert owns
    say(f"grouped gemm E={E} counts={counts} N={N} K={K} g={g}")
    X = wl.gen_activations(M, K, 600 + M, 601)
    X8, sx = oracle.quant_sym_rows(X, 127)
    refs = [oracle.w4a8_pack(wl.gen_weights(N, K, 610 + e), g) for e in range(E)]
    pk = {"wq": to_dev(np.concatenate([r["wq"].ravel() for r in refs])),
          "s_u8": to_dev(np.concatenate([r["s_panels"] for r in refs])),
          "a_u8": to_dev(np.concatenate([r["a_panels"] for r in refs])),
          "sw": to_dev(np.concatenate([r["sw"] for r in refs])),
          "N": N, "K": K, "group": g, "E": E}
    off_d = to_dev(offs)
    Yi = poison((M, N), torch.int32)
    w4.gemm_grouped(to_dev(X8), to_dev(sx), off_d, pk, max(counts), out_type=w4.OUT_I32, out=Yi)
    Yh = poison((M, N), torch.float16)
    w4.gemm_grouped(to_dev(X8), to_dev(sx), off_d, pk, max(counts), out_type=w4.OUT_F16, out=Yh)
    yi, yh = host(Yi), host(Yh.view(torch.int16)).view(np.uint16)
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        if r1 == r0:
            continue
        acc, y, _ = oracle.w4a8_gemm(X8[r0:r1], sx[r0:r1], refs[e], g)
        np.testing.assert_array_equal(yi[r0:r1], acc)
        assert f16_ulp_diff(yh[r0:r1], y).max() <= 1
    assert np.all(yi[offs[-1]:].view(np.uint32) == 0xABABABAB)   # untouched


@pytest.mark.parametrize("N", [128, 256])   # streamed kernel / 128-row tiles
def test_grouped_bad_offsets_clamped(N):
    """Offsets out of order, negative and past M: each expert's rows are
    clamped to [0, M] (lo = clamp(off[e]), hi = clamp(max(off[e+1], lo))), as
    the header states, so bad offsets only leave rows unwritten.  Here expert
    0 and 3 come out empty, experts 1 and 2 own rows 5..59 and 60..99, and
    rows 0..4 stay untouched."""
    M, K, g, E = 100, 512, 128, 4
    offs = np.array([10, 5, 60, 200, -3], np.int32)
    owned = {1: (5, 60), 2: (60, 100)}
    say(f"grouped gemm, bad offsets {offs.tolist()} M={M} N={N}")
    X = wl.gen_activations(M, K, 700, 701)
    X8, sx = oracle.quant_sym_rows(X, 127)
    refs = [oracle.w4a8_pack(wl.gen_weights(N, K, 710 + e), g) for e in range(E)]
    pk = {"wq": to_dev(np.concatenate([r["wq"].ravel() for r in refs])),
          "s_u8": to_dev(np.concatenate([r["s_panels"] for r in refs])),
          "a_u8": to_dev(np.concatenate([r["a_panels"] for r in refs])),
          "sw": to_dev(np.concatenate([r["sw"] for r in refs])),
          "N": N, "K": K, "group": g, "E": E}
    Yi = poison((M, N), torch.int32)
    w4.gemm_grouped(to_dev(X8), to_dev(sx), to_dev(offs), pk, M, out_type=w4.OUT_I32, out=Yi)
    yi = host(Yi)
    for e, (r0, r1) in owned.items():
        acc, _, _ = oracle.w4a8_gemm(X8[r0:r1], sx[r0:r1], refs[e], g)
        np.testing.assert_array_equal(yi[r0:r1], acc)
    assert np.all(yi[:5].view(np.uint32) == 0xABABABAB)   # no expert owns rows 0..4


@pytest.mark.parametrize("M,N,K,splits", [(600, 4352, 3072, 3), (300, 4352, 5120, 5),
                                           (500, 2304, 7168, 7), (100, 256, 16384, 16),
                                           (640, 2048, 6272, 6), (100, 6912, 9216, 9),
                                           (128, 6144, 10368, 10), (64, 5632, 11264, 11),
                                           (128, 5120, 12416, 12), (128, 4864, 13312, 13),
                                           (128, 4608, 14464, 14), (128, 4352, 15360, 15)])
def test_split_counts_any_integer(M, N, K, splits):
    """The split-K plan fills one wave of CUs with any integer split count
    (the reduction is built once per count, 2 to 16; the even counts here
    keep their splits, since K parts would read X again for more bytes than
    the partials): int32 results bit-exact against the oracle on sampled
    rows (the oracle quantises per row, so a row sample is exact) and
    against the streamed kernel on every element."""
    assert w4.workspace_size(M, N, K) == splits * M * N * 4
    g = 128
    say(f"w4a8 split-K {splits} M={M} N={N} K={K}")
    W = wl.gen_weights(N, K, 3000 + splits)
    X = wl.gen_activations(M, K, 3001 + splits, 3002)
    pk_ref = oracle.w4a8_pack(W, g)
    X8, sx = oracle.quant_sym_rows(X, 127)
    pk = {"wq": to_dev(pk_ref["wq"]), "s_u8": to_dev(pk_ref["s_panels"]),
          "a_u8": to_dev(pk_ref["a_panels"]), "sw": to_dev(pk_ref["sw"]),
          "N": N, "K": K, "group": g}
    Yi = poison((M, N), torch.int32)
    w4.gemm(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_I32, out=Yi)
    got = host(Yi)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(splits).choice(M, 6)]))
    acc, _, _ = oracle.w4a8_gemm(X8[rows], sx[rows], pk_ref, g)
    np.testing.assert_array_equal(got[rows], acc)
    Ys = poison((M, N), torch.int32)
    w4.gemm(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_I32, splitk=1, out=Ys)
    np.testing.assert_array_equal(got, host(Ys))


def test_workspace_shared_across_split_calls():
    """One workspace serves a sequence of split-K calls of different shapes
    and kinds (W4A8, FP8, W8A8) ordered on one stream: whatever one call
    leaves in it does not reach the next call's results."""
    shapes = [(128, 512, 4096, 128), (100, 256, 2048, 64), (200, 1024, 8192, 128)]
    need = max(w4.workspace_size(M, N, K) for M, N, K, _ in shapes)
    ws = poison((need,), torch.uint8)
    for i, (M, N, K, g) in enumerate(shapes):
        say(f"shared workspace, call {i}: M={M} N={N} K={K} g={g}")
        assert w4.workspace_size(M, N, K) > 0
        X8, sx, pk, acc, y = _small_problem(M, N, K, g, 3300 + i)
        Yi = poison((M, N), torch.int32)
        w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi, workspace=ws)
        np.testing.assert_array_equal(host(Yi), acc)
        # FP8 split call on the same workspace
        W = wl.gen_weights(N, K, 3300 + i)
        Xf = wl.gen_activations(M, K, 3301 + i, 3302 + i)
        Xe, sxe = oracle.quant_rows_e4m3(Xf)
        pf = oracle.w4fp8_pack(W)
        pkf = {"wq": to_dev(pf["wq"]), "sw": to_dev(pf["sw"]), "N": N, "K": K}
        Yf = poison((M, N), torch.float32)
        w4.gemm_fp8(to_dev(Xe), to_dev(sxe), pkf, out_type=w4.OUT_F32, out=Yf, workspace=ws)
        ref, _ = oracle.w4fp8_ref(Xe, sxe, pf["q"], pf["sw"])
        assert rel_fro(host(Yf), ref) <= 1e-3
        # W8A8 split call
        ref8 = oracle.w8a8_pack(W)
        acc8, _, _ = oracle.w8a8_gemm(host(X8), host(sx), ref8)
        pk8 = {"wq8": to_dev(ref8["wq8"]), "sw": to_dev(ref8["sw"]), "N": N, "K": K}
        Yi = poison((M, N), torch.int32)
        w4.gemm_w8a8(X8, sx, pk8, out_type=w4.OUT_I32, out=Yi, workspace=ws)
        np.testing.assert_array_equal(host(Yi), acc8)


def test_workspace_too_small_is_rejected():
    M, N, K = 128, 512, 4096
    X8, sx, pk, acc, y = _small_problem(M, N, K, 128, 3)
    need = w4.workspace_size(M, N, K)
    small = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(w4.W4A8Error) as ei:
        w4.gemm(X8, sx, pk, workspace=small)
    assert ei.value.status == 4


def test_splitk_invariance_and_determinism():
    say("w4a8 split-K sweep M=16 N=256 K=2048")
    X8, sx, pk, acc, _ = _small_problem(16, 256, 2048, 64, 77)
    outs = []
    for sk in (1, 2, 4, 8, 16, 0, 0):
        Y = poison((16, 256), torch.int32)
        w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, splitk=sk, out=Y)
        outs.append(host(Y))
    for o in outs:
        np.testing.assert_array_equal(o, acc)


def test_empty_problem_touches_nothing():
    X8, sx, pk, acc, _ = _small_problem(4, 64, 256, 64, 5)
    Y = poison((4, 64), torch.float16)
    w4.gemm(X8[:0], sx[:0], pk, out=Y[:0])
    assert np.all(host(Y.view(torch.uint8)) == 0xAB)


# ------------------------------------------------------ W4FP8 GEMM ---------
@pytest.mark.parametrize("M", [1, 16, 37])
def test_w4fp8_gemm_parity(M):
    N, K = 128, 1024
    say(f"w4fp8 gemm M={M} N={N} K={K}")
    W = wl.gen_weights(N, K, 400 + M)
    X = wl.gen_activations(M, K, 401 + M, 402)
    pk_ref = oracle.w4fp8_pack(W)
    X8, sx = oracle.quant_rows_e4m3(X)
    ref, _ = oracle.w4fp8_ref(X8, sx, pk_ref["q"], pk_ref["sw"])
    pk = {"wq": to_dev(pk_ref["wq"]), "sw": to_dev(pk_ref["sw"]), "N": N, "K": K}
    Yf = poison((M, N), torch.float32)
    w4.gemm_fp8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F32, out=Yf)
    err = rel_fro(host(Yf), ref)
    say(f"  f32 vs fp64 rel fro {err:.3e}")
    assert err <= 1e-3
    Yb = poison((M, N), torch.bfloat16)
    w4.gemm_fp8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_BF16, out=Yb)
    got = bf16_bits_of(Yb)
    want = oracle.round_bf16(ref)
    gv = (got.astype(np.uint32) << 16).view(np.float32)
    wv = (want.astype(np.uint32) << 16).view(np.float32)
    err_b = rel_fro(gv, wv)
    say(f"  bf16 vs bf16(fp64) rel fro {err_b:.3e}; vs fp64 {rel_fro(gv, ref):.3e}")
    assert err_b <= 1e-3
    _check_fp8_outputs(host(Yf), got, ref, _fp8_bound(X8, sx, pk_ref["q"], pk_ref["sw"]))


def _fp8_bound(X8, sx, q, sw):
    """Elementwise bound for the FP8 paths against the exact value.

    The products x_k q_k are exact, but the gfx950 FP8 matrix instruction
    does not add them as IEEE float32: next to a large product of the same
    instruction, smaller ones lose low-order bits (measured on crafted rows:
    448 followed by 255 terms of 2^-9 gives 448.484375, not 448.498047; the
    tile and streamed kernels agree bit for bit).  Bound: 2^-10 of the
    largest |product| of every 64-column block (taken as max|x| * max|q| of
    the block; the largest loss seen is about 2^-13 of it), plus float32
    summation across blocks, (K + 2) u sum_k |x_k q_k| with u = 2^-24, both
    scaled by sx sw.  A wrong operand index or a dropped K-chunk is an error
    of whole average products, far above this; exact indexing is pinned
    separately by the integer-valued test."""
    return _fp8_bound_w(X8, sx, np.abs(q.astype(np.float64)), sw)


def _fp8_bound_w(X8, sx, qd, sw):
    """_fp8_bound for weight magnitudes qd [N][K] (any exact e4m3 values)
    and a column scale sw [N] (a vector, or the tensor scale broadcast)."""
    xd = np.abs(oracle.e4m3_decode(X8))
    M, K = X8.shape
    absum = xd @ qd.T
    xm = xd.reshape(M, K // 64, 64).max(axis=2)
    qm = qd.reshape(qd.shape[0], K // 64, 64).max(axis=2)
    blk = xm @ qm.T
    sw = np.broadcast_to(np.asarray(sw, np.float64), (qd.shape[0],))
    return ((K + 2) * 2.0 ** -24 * absum + 2.0 ** -10 * blk) \
        * np.asarray(sx, np.float64)[:, None] * sw[None, :]


def _check_fp8_outputs(yf, yb_bits, ref, bound):
    """float32 output inside the bound elementwise; bfloat16 output inside it
    plus one bfloat16 rounding (unit roundoff 2^-8); both within relative
    Frobenius 1e-3 of the double reference (the bfloat16 one of the
    bfloat16-rounded reference)."""
    yf = np.asarray(yf, np.float64)
    assert np.all(np.abs(yf - ref) <= bound + 1e-30)
    assert rel_fro(yf, ref) <= 1e-3
    gv = (yb_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    lim = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref) + 1e-30
    assert np.all(np.abs(gv - ref) <= lim)
    wv = (oracle.round_bf16(ref).astype(np.uint32) << 16).view(np.float32)
    assert rel_fro(gv, wv) <= 1e-3


@pytest.mark.parametrize("M,N,K", [(16, 128, 1024), (100, 256, 1024), (300, 512, 2048),
                                   (128, 256, 4096), (100, 256, 640), (300, 512, 1152),
                                   (16, 128, 128), (100, 256, 128)])
def test_w4fp8_integer_valued_exact(M, N, K):
    """Integer activations in [-16, 16] (exact in e4m3) times |q| <= 7: every
    product is an integer <= 112 and every partial sum an integer below
    2^24, so any summation order and the instruction's internal alignment
    are exact -- the float32 output (sx = sw = 1) must equal the integer sum
    bit for bit.  Pins operand layout, K indexing and split-K partials."""
    say(f"w4fp8 integer-valued exact M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    Xi = rng.integers(-16, 17, size=(M, K)).astype(np.float64)
    q = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    X8 = oracle.e4m3_encode(Xi)
    np.testing.assert_array_equal(oracle.e4m3_decode(X8), Xi)
    wq = oracle.pack_nibbles(oracle.int4_sm_codes(q))
    exact = Xi.astype(np.int64) @ q.astype(np.int64).T
    pk = {"wq": to_dev(wq), "sw": to_dev(np.ones(N, np.float32)), "N": N, "K": K}
    ones = to_dev(np.ones(M, np.float32))
    for sk in (0, 1):
        Y = poison((M, N), torch.float32)
        w4.gemm_fp8(to_dev(X8), ones, pk, out_type=w4.OUT_F32, splitk=sk, out=Y)
        np.testing.assert_array_equal(host(Y), exact.astype(np.float32))


# Matrix-core tile path (M >= 64, N % 256 == 0): ragged M, several tiles in
# both directions, one and two K-steps per split, and planned split-K with
# float32 partials (M=128, K=4096: one tile, four splits; then 16, 9, 13 and
# 6 splits, each count a reduction of its own).
@pytest.mark.parametrize("M,N,K", [(64, 256, 640), (512, 1024, 896), (300, 512, 1152),
                                   (64, 256, 1024), (100, 256, 1024), (256, 512, 2048),
                                   (300, 512, 1024), (513, 256, 2048), (128, 256, 4096),
                                   (100, 512, 2048), (1024, 1024, 256), (100, 256, 16384),
                                   (100, 6912, 9216), (128, 4864, 13312), (640, 2048, 6272)])
def test_w4fp8_tile_parity(M, N, K):
    say(f"w4fp8 tile gemm M={M} N={N} K={K} workspace={w4.workspace_size(M, N, K)}")
    W = wl.gen_weights(N, K, 500 + M + N)
    X = wl.gen_activations(M, K, 501 + M, 502)
    pk_ref = oracle.w4fp8_pack(W)
    X8, sx = oracle.quant_rows_e4m3(X)
    ref, _ = oracle.w4fp8_ref(X8, sx, pk_ref["q"], pk_ref["sw"])
    bound = _fp8_bound(X8, sx, pk_ref["q"], pk_ref["sw"])
    pk = {"wq": to_dev(pk_ref["wq"]), "sw": to_dev(pk_ref["sw"]), "N": N, "K": K}
    Yf = poison((M, N), torch.float32)
    w4.gemm_fp8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F32, out=Yf)
    Yb = poison((M, N), torch.bfloat16)
    w4.gemm_fp8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_BF16, out=Yb)
    yf = host(Yf)
    say(f"  f32 rel fro {rel_fro(yf, ref):.3e}; max |err|/bound "
        f"{np.max(np.abs(yf - ref) / (bound + 1e-30)):.3f}")
    _check_fp8_outputs(yf, bf16_bits_of(Yb), ref, bound)
    # the streamed kernel (forced by splitk) meets the same bound
    Ys = poison((M, N), torch.float32)
    w4.gemm_fp8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F32, splitk=1, out=Ys)
    assert np.all(np.abs(host(Ys) - ref) <= bound + 1e-30)


# Large FP8 grids (at least 256 tiles of 256 rows: M x N = 4096 x 4096 and
# more) with short K, which run 128-row tiles two per CU.  K = 384: odd
# K-step count (the tail step); M = 4000: ragged last row tile.
@pytest.mark.parametrize("M,N,K", [(4000, 4096, 384), (4096, 4096, 512)])
def test_w4fp8_large_grid(M, N, K):
    say(f"w4fp8 large grid M={M} N={N} K={K} workspace={w4.workspace_size(M, N, K)}")
    assert w4.workspace_size(M, N, K) == 0
    # integer-valued operands: exact in any summation order, bit for bit
    rng = np.random.default_rng(M + K)
    Xi = rng.integers(-16, 17, size=(M, K)).astype(np.float64)
    q = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    X8 = oracle.e4m3_encode(Xi)
    exact = Xi.astype(np.int64) @ q.astype(np.int64).T
    pk = {"wq": to_dev(oracle.pack_nibbles(oracle.int4_sm_codes(q))),
          "sw": to_dev(np.ones(N, np.float32)), "N": N, "K": K}
    Y = poison((M, N), torch.float32)
    w4.gemm_fp8(to_dev(X8), to_dev(np.ones(M, np.float32)), pk, out_type=w4.OUT_F32, out=Y)
    np.testing.assert_array_equal(host(Y), exact.astype(np.float32))
    # realistic data against the double reference, both output types
    W = wl.gen_weights(N, K, 510 + K)
    X = wl.gen_activations(M, K, 511 + K, 512)
    pk_ref = oracle.w4fp8_pack(W)
    X8, sx = oracle.quant_rows_e4m3(X)
    ref, _ = oracle.w4fp8_ref(X8, sx, pk_ref["q"], pk_ref["sw"])
    bound = _fp8_bound(X8, sx, pk_ref["q"], pk_ref["sw"])
    pk = {"wq": to_dev(pk_ref["wq"]), "sw": to_dev(pk_ref["sw"]), "N": N, "K": K}
    Yf = poison((M, N), torch.float32)
    w4.gemm_fp8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F32, out=Yf)
    Yb = poison((M, N), torch.bfloat16)
    w4.gemm_fp8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_BF16, out=Yb)
    yf = host(Yf)
    say(f"  f32 rel fro {rel_fro(yf, ref):.3e}; max |err|/bound "
        f"{np.max(np.abs(yf - ref) / (bound + 1e-30)):.3f}")
    _check_fp8_outputs(yf, bf16_bits_of(Yb), ref, bound)


def test_fp8_workspace_too_small_is_rejected():
    M, N, K = 128, 256, 4096
    need = w4.workspace_size(M, N, K)
    assert need > 0
    X8 = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    sx = torch.ones(M, dtype=torch.float32, device=DEV)
    pk = {"wq": torch.zeros(N * K // 2, dtype=torch.uint8, device=DEV),
          "sw": torch.ones(N, dtype=torch.float32, device=DEV), "N": N, "K": K}
    small = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(w4.W4A8Error) as ei:
        w4.gemm_fp8(X8, sx, pk, workspace=small)
    assert ei.value.status == 4


# ------------------------------------------------ W8A8 comparison ---------
@pytest.mark.parametrize("N,K", [(64, 256), (320, 1152), (256, 640)])
def test_w8a8_pack_parity(N, K):
    say(f"w8a8 pack N={N} K={K}")
    W = wl.gen_weights(N, K, 1100 + N)
    W[2, :] = 0.0
    ref = oracle.w8a8_pack(W)
    pk = w4.pack_w8(to_dev(W))
    np.testing.assert_array_equal(host(pk["wq8"]), ref["wq8"])
    np.testing.assert_array_equal(host(pk["sw"]).view(np.uint32), ref["sw"].view(np.uint32))


@pytest.mark.parametrize("M,N,K,sk", [(1, 128, 640, 0), (5, 64, 512, 0), (16, 448, 1024, 0),
                                      (33, 256, 512, 0), (64, 256, 640, 0), (100, 512, 1024, 0),
                                      (300, 512, 1152, 0), (513, 256, 512, 0),
                                      (128, 256, 4096, 0), (100, 256, 896, 2), (257, 1024, 256, 0),
                                      (16, 10240, 1024, 0), (16, 8192, 512, 0),
                                      (40, 28672, 512, 0), (16, 256, 128, 0),
                                      (128, 512, 128, 0), (300, 256, 128, 0)])
def test_w8a8_gemm_parity(M, N, K, sk):
    """int32 bit-exact and fp16 within 1 ulp against the oracle: streamed
    kernel (M < 64, N % 256 != 0, or forced by splitk; 1, 2, 4 and 7 tiles
    per workgroup), tile kernels with 128-row tiles, ragged M, odd K-step
    counts and planned split-K."""
    say(f"w8a8 gemm M={M} N={N} K={K} splitk={sk} workspace={w4.workspace_size(M, N, K, sk)}")
    W = wl.gen_weights(N, K, 1200 + M + N)
    X = wl.gen_activations(M, K, 1201 + M, 1202)
    ref = oracle.w8a8_pack(W)
    X8, sx = oracle.quant_sym_rows(X, 127)
    acc, y, _ = oracle.w8a8_gemm(X8, sx, ref)
    pk = {"wq8": to_dev(ref["wq8"]), "sw": to_dev(ref["sw"]), "N": N, "K": K}
    Yi = poison((M, N), torch.int32)
    w4.gemm_w8a8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_I32, splitk=sk, out=Yi)
    np.testing.assert_array_equal(host(Yi), acc)
    Yh = poison((M, N), torch.float16)
    w4.gemm_w8a8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F16, splitk=sk, out=Yh)
    d = f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y)
    assert d.max() <= 1
    if sk == 0 and M >= 64:  # the streamed kernel agrees
        Ys = poison((M, N), torch.int32)
        w4.gemm_w8a8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_I32, splitk=1, out=Ys)
        np.testing.assert_array_equal(host(Ys), acc)


def test_w8a8_large_grid():
    """W8A8 on a large short-K grid (128-row tiles two per CU on the
    16 x 16 x 64 tile kernel): int32 bit-exact
    against the oracle on sampled rows and against the streamed kernel on
    every element; fp16 within 1 ulp on the sampled rows."""
    M, N, K = 4096, 4096, 384
    assert w4.workspace_size(M, N, K) == 0
    say(f"w8a8 large grid M={M} N={N} K={K}")
    W = wl.gen_weights(N, K, 1301)
    X = wl.gen_activations(M, K, 1302, 1303)
    ref = oracle.w8a8_pack(W)
    X8, sx = oracle.quant_sym_rows(X, 127)
    pk = {"wq8": to_dev(ref["wq8"]), "sw": to_dev(ref["sw"]), "N": N, "K": K}
    Yi = poison((M, N), torch.int32)
    w4.gemm_w8a8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_I32, out=Yi)
    Yh = poison((M, N), torch.float16)
    w4.gemm_w8a8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F16, out=Yh)
    got = host(Yi)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(9).choice(M, 8)]))
    acc, y, _ = oracle.w8a8_gemm(X8[rows], sx[rows], ref)
    np.testing.assert_array_equal(got[rows], acc)
    d = f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16)[rows], y)
    assert d.max() <= 1
    Ys = poison((M, N), torch.int32)
    w4.gemm_w8a8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_I32, splitk=1, out=Ys)
    np.testing.assert_array_equal(got, host(Ys))


# ----------------------------- folded per-group FP8 (FireQ-style) ----------
def _fp8g_weights(N, K, g, seed):
    """Normal(0, 0.02) weights with one all-zero row and one all-zero group
    (scale 1, codes 0) and a tiny-valued group (folded weights in the e4m3
    subnormal range)."""
    W = wl.gen_weights(N, K, seed)
    W[3, :] = 0.0
    W[5, g:2 * g] = 0.0
    W[7, :g] *= np.float32(1e-4)
    return W


def _fp8g_device(pk_ref, N, K, g):
    return {"wq": to_dev(pk_ref["wq"]), "fsc": to_dev(np.ascontiguousarray(pk_ref["f"].T)),
            "tscale": to_dev(np.array([pk_ref["t"]], np.float32)), "N": N, "K": K, "group": g}


@pytest.mark.parametrize("N,K,g", [(64, 256, 64), (320, 1024, 128), (256, 1152, 64)])
def test_fp8g_pack_parity(N, K, g):
    """Device packing bit-exact: codes, group-major folded factors, t."""
    say(f"w4fp8g pack N={N} K={K} g={g}")
    W = _fp8g_weights(N, K, g, 600 + N + K)
    ref = oracle.w4fp8g_pack(W, g)
    pk = w4.pack_fp8g(to_dev(W), group=g)
    np.testing.assert_array_equal(host(pk["wq"]), ref["wq"])
    np.testing.assert_array_equal(host(pk["fsc"]).view(np.uint32),
                                  np.ascontiguousarray(ref["f"].T).view(np.uint32))
    assert host(pk["tscale"]).view(np.uint32)[0] == np.float32(ref["t"]).view(np.uint32)


@pytest.mark.parametrize("K,N,g,sk", [(256, 256, 64, 0), (512, 512, 128, 0), (384, 256, 64, 0),
                                      (256, 192, 128, 0), (512, 256, 64, 1),
                                      (384, 128, 128, 2)])
def test_fp8g_folded_weights_exact(K, N, g, sk):
    """X = identity (M = K rows, e4m3 1.0, sx = 1): output row k, column n is
    the single product w8[n][k] * 1, so the float32 output must equal
    float32(w8 * t) bit for bit -- every folded e4m3 weight the kernel forms
    in registers is checked against the oracle's encoding (tile kernel for
    N % 256 == 0, streamed kernel otherwise or when splitk forces it)."""
    say(f"w4fp8g folded weights K={K} N={N} g={g} splitk={sk}")
    W = _fp8g_weights(N, K, g, 700 + K + N)
    ref = oracle.w4fp8g_pack(W, g)
    X8 = np.zeros((K, K), np.uint8)
    np.fill_diagonal(X8, 0x38)
    sx = np.ones(K, np.float32)
    want = (oracle.e4m3_decode(ref["w8"]).T.astype(np.float32) * np.float32(ref["t"]))
    Y = poison((K, N), torch.float32)
    w4.gemm_fp8g(to_dev(X8), to_dev(sx), _fp8g_device(ref, N, K, g), out_type=w4.OUT_F32,
                 splitk=sk, out=Y)
    np.testing.assert_array_equal(host(Y).view(np.uint32), want.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("M,N,K,g", [(1, 256, 1024, 128), (16, 512, 2048, 64),
                                     (37, 128, 640, 128), (64, 256, 640, 64),
                                     (300, 512, 1152, 128), (513, 256, 2048, 64),
                                     (128, 256, 4096, 128), (100, 512, 2048, 64),
                                     (1024, 1024, 256, 128)])
def test_fp8g_gemm_parity(M, N, K, g):
    """Realistic weights and activations against the oracle's double result:
    elementwise inside the FP8 bound (with |w8| in place of |q| and t as the
    column scale), relative Frobenius <= 1e-3; both output types; the
    streamed kernel forced by splitk meets the same bound.  Covers streamed
    and tile kernels, ragged M, odd K-step counts and planned split-K."""
    say(f"w4fp8g gemm M={M} N={N} K={K} g={g} workspace={w4.workspace_size(M, N, K)}")
    W = _fp8g_weights(N, K, g, 800 + M + N)
    X = wl.gen_activations(M, K, 801 + M, 802)
    ref_pk = oracle.w4fp8g_pack(W, g)
    X8, sx = oracle.quant_rows_e4m3(X)
    ref, _ = oracle.w4fp8g_ref(X8, sx, ref_pk["w8"], ref_pk["t"])
    bound = _fp8_bound_w(X8, sx, np.abs(oracle.e4m3_decode(ref_pk["w8"])), ref_pk["t"])
    pk = _fp8g_device(ref_pk, N, K, g)
    Yf = poison((M, N), torch.float32)
    w4.gemm_fp8g(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F32, out=Yf)
    Yb = poison((M, N), torch.bfloat16)
    w4.gemm_fp8g(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_BF16, out=Yb)
    yf = host(Yf)
    say(f"  f32 rel fro {rel_fro(yf, ref):.3e}; max |err|/bound "
        f"{np.max(np.abs(yf - ref) / (bound + 1e-30)):.3f}")
    _check_fp8_outputs(yf, bf16_bits_of(Yb), ref, bound)
    Ys = poison((M, N), torch.float32)
    w4.gemm_fp8g(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F32, splitk=1, out=Ys)
    assert np.all(np.abs(host(Ys) - ref) <= bound + 1e-30)


# The FP8 streamed kernel at 4 tiles per workgroup (N = 10240, one 16-row
# block per workgroup), two row blocks at 4, 2 and 1 tiles (the last with a
# second workgroup along M whose blocks lie partly and wholly past M) and
# four row blocks at 2 tiles, per-channel and folded: integer-valued
# operands bit for bit, realistic data against the double reference.
@pytest.mark.parametrize("M,N,K", [(16, 10240, 1024), (20, 10240, 640), (24, 8192, 1024),
                                   (48, 2048, 1024), (40, 28672, 512)])
def test_fp8_stream_widths(M, N, K):
    say(f"w4fp8 streamed kernel widths: M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N)
    Xi = rng.integers(-16, 17, size=(M, K)).astype(np.float64)
    q = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    exact = Xi.astype(np.int64) @ q.astype(np.int64).T
    pk = {"wq": to_dev(oracle.pack_nibbles(oracle.int4_sm_codes(q))),
          "sw": to_dev(np.ones(N, np.float32)), "N": N, "K": K}
    Y = poison((M, N), torch.float32)
    w4.gemm_fp8(to_dev(oracle.e4m3_encode(Xi)), to_dev(np.ones(M, np.float32)), pk,
                out_type=w4.OUT_F32, out=Y)
    np.testing.assert_array_equal(host(Y), exact.astype(np.float32))
    W = wl.gen_weights(N, K, 530 + M)
    X = wl.gen_activations(M, K, 531 + M, 532)
    X8, sx = oracle.quant_rows_e4m3(X)
    pk_ref = oracle.w4fp8_pack(W)
    ref, _ = oracle.w4fp8_ref(X8, sx, pk_ref["q"], pk_ref["sw"])
    bound = _fp8_bound(X8, sx, pk_ref["q"], pk_ref["sw"])
    pk = {"wq": to_dev(pk_ref["wq"]), "sw": to_dev(pk_ref["sw"]), "N": N, "K": K}
    Yf = poison((M, N), torch.float32)
    w4.gemm_fp8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F32, out=Yf)
    Yb = poison((M, N), torch.bfloat16)
    w4.gemm_fp8(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_BF16, out=Yb)
    _check_fp8_outputs(host(Yf), bf16_bits_of(Yb), ref, bound)
    g = 128
    Wg = _fp8g_weights(N, K, g, 540 + M)
    ref_pk = oracle.w4fp8g_pack(Wg, g)
    refg, _ = oracle.w4fp8g_ref(X8, sx, ref_pk["w8"], ref_pk["t"])
    boundg = _fp8_bound_w(X8, sx, np.abs(oracle.e4m3_decode(ref_pk["w8"])), ref_pk["t"])
    pkg = _fp8g_device(ref_pk, N, K, g)
    Yf = poison((M, N), torch.float32)
    w4.gemm_fp8g(to_dev(X8), to_dev(sx), pkg, out_type=w4.OUT_F32, out=Yf)
    Yb = poison((M, N), torch.bfloat16)
    w4.gemm_fp8g(to_dev(X8), to_dev(sx), pkg, out_type=w4.OUT_BF16, out=Yb)
    _check_fp8_outputs(host(Yf), bf16_bits_of(Yb), refg, boundg)


# Folded format on large short-K grids (128-row tiles two per CU): identity X
# with M = K = 4096 checks every folded e4m3 weight bit for bit; realistic
# data with ragged M and an odd K-step count against the double reference.
@pytest.mark.parametrize("g", [64, 128])
def test_fp8g_large_grid(g):
    N = K = 4096
    say(f"w4fp8g large grid, identity X: K={K} N={N} g={g}")
    assert w4.workspace_size(K, N, K) == 0
    W = _fp8g_weights(N, K, g, 710 + g)
    ref = oracle.w4fp8g_pack(W, g)
    X8 = np.zeros((K, K), np.uint8)
    np.fill_diagonal(X8, 0x38)
    want = (oracle.e4m3_decode(ref["w8"]).T.astype(np.float32) * np.float32(ref["t"]))
    Y = poison((K, N), torch.float32)
    w4.gemm_fp8g(to_dev(X8), to_dev(np.ones(K, np.float32)), _fp8g_device(ref, N, K, g),
                 out_type=w4.OUT_F32, out=Y)
    np.testing.assert_array_equal(host(Y).view(np.uint32), want.astype(np.float32).view(np.uint32))
    del Y
    M, K = 4000, 384
    say(f"w4fp8g large grid M={M} N={N} K={K} g={g}")
    W = _fp8g_weights(N, K, g, 720 + g)
    X = wl.gen_activations(M, K, 721, 722)
    ref_pk = oracle.w4fp8g_pack(W, g)
    X8, sx = oracle.quant_rows_e4m3(X)
    ref, _ = oracle.w4fp8g_ref(X8, sx, ref_pk["w8"], ref_pk["t"])
    bound = _fp8_bound_w(X8, sx, np.abs(oracle.e4m3_decode(ref_pk["w8"])), ref_pk["t"])
    pk = _fp8g_device(ref_pk, N, K, g)
    Yf = poison((M, N), torch.float32)
    w4.gemm_fp8g(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F32, out=Yf)
    Yb = poison((M, N), torch.bfloat16)
    w4.gemm_fp8g(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_BF16, out=Yb)
    _check_fp8_outputs(host(Yf), bf16_bits_of(Yb), ref, bound)


def test_256_row_tiles_long_k():
    """Plans with more than 64 K-steps per workgroup keep 256-row tiles
    (4000 x 4096 x 8320: 65 K-steps, the odd tail step, a ragged last row
    tile), for all four tile GEMMs.  Sampled rows against the oracle (it
    quantises per row, so a row sample is exact): W4A8 and W8A8 int32
    bit-exact and fp16 within 1 ulp; FP8 per-channel and folded g = 128
    inside the FP8 bound."""
    M, N, K, g = 4000, 4096, 8320, 128
    assert w4.workspace_size(M, N, K) == 0
    say(f"256-row tiles, long K: M={M} N={N} K={K}")
    rows = np.unique(np.concatenate([[0, 255, 256, 3839, 3840, M - 1],
                                     np.random.default_rng(17).choice(M, 10, replace=False)]))
    W = wl.gen_weights(N, K, 1401)
    X = wl.gen_activations(M, K, 1402, 1403)
    # W4A8
    ref = oracle.w4a8_pack(W, g)
    X8, sx = oracle.quant_sym_rows(X, 127)
    pk = {"wq": to_dev(ref["wq"]), "s_u8": to_dev(ref["s_panels"]),
          "a_u8": to_dev(ref["a_panels"]), "sw": to_dev(ref["sw"]), "N": N, "K": K, "group": g}
    Yi = poison((M, N), torch.int32)
    w4.gemm(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_I32, out=Yi)
    Yh = poison((M, N), torch.float16)
    w4.gemm(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F16, out=Yh)
    acc, y, _ = oracle.w4a8_gemm(X8[rows], sx[rows], ref, g)
    np.testing.assert_array_equal(host(Yi)[rows], acc)
    assert f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16)[rows], y).max() <= 1
    del Yi, Yh, pk
    # W8A8
    ref8 = oracle.w8a8_pack(W)
    pk8 = {"wq8": to_dev(ref8["wq8"]), "sw": to_dev(ref8["sw"]), "N": N, "K": K}
    Yi = poison((M, N), torch.int32)
    w4.gemm_w8a8(to_dev(X8), to_dev(sx), pk8, out_type=w4.OUT_I32, out=Yi)
    acc8, _, _ = oracle.w8a8_gemm(X8[rows], sx[rows], ref8)
    np.testing.assert_array_equal(host(Yi)[rows], acc8)
    del Yi, pk8
    # FP8, per-channel and folded
    Xe, sxe = oracle.quant_rows_e4m3(X)
    pf = oracle.w4fp8_pack(W)
    pkf = {"wq": to_dev(pf["wq"]), "sw": to_dev(pf["sw"]), "N": N, "K": K}
    Yf = poison((M, N), torch.float32)
    w4.gemm_fp8(to_dev(Xe), to_dev(sxe), pkf, out_type=w4.OUT_F32, out=Yf)
    reff, _ = oracle.w4fp8_ref(Xe[rows], sxe[rows], pf["q"], pf["sw"])
    bound = _fp8_bound(Xe[rows], sxe[rows], pf["q"], pf["sw"])
    yf = host(Yf)[rows].astype(np.float64)
    assert np.all(np.abs(yf - reff) <= bound + 1e-30) and rel_fro(yf, reff) <= 1e-3
    pg = oracle.w4fp8g_pack(W, g)
    Yf = poison((M, N), torch.float32)
    w4.gemm_fp8g(to_dev(Xe), to_dev(sxe), _fp8g_device(pg, N, K, g), out_type=w4.OUT_F32, out=Yf)
    refg, _ = oracle.w4fp8g_ref(Xe[rows], sxe[rows], pg["w8"], pg["t"])
    boundg = _fp8_bound_w(Xe[rows], sxe[rows], np.abs(oracle.e4m3_decode(pg["w8"])), pg["t"])
    yg = host(Yf)[rows].astype(np.float64)
    assert np.all(np.abs(yg - refg) <= boundg + 1e-30) and rel_fro(yg, refg) <= 1e-3


# The 256-row plan of the 16 x 16 x 64 kernel (the one the M = 4096 Llama-2-70B
# shapes run), every output element against the oracle, outputs poisoned:
# short K with an even (2) and odd (3) K-step count on a grid of 1024 tiles
# (four waves, so 256-row tiles stay), and long K with 65 (odd, the padding
# step) and 66 (even) K-steps; 4000 rows leave a ragged last row tile.  The
# W8A8 comparison runs the same plan.  These are the cases where a missed
# wait state in the hand-placed matrix-core schedule would show.  Two more
# long-K cases with rows past M in the last row tile: 304 tiles (66 K-steps)
# and 512 tiles (65 K-steps).
_PLAN256 = [(4096, 16384, 256, 64, True), (4096, 16384, 384, 128, True),
            (4000, 4096, 8320, 128, True), (4096, 4096, 8448, 64, False),
            (4000, 4864, 8448, 128, True), (4000, 8192, 8320, 64, False)]


@pytest.mark.parametrize("M,N,K,g,w8", _PLAN256)
def test_256_row_plan_every_element(M, N, K, g, w8):
    assert w4.workspace_size(M, N, K) == 0
    say(f"256-row 16x16x64 plan, every element: M={M} N={N} K={K} g={g}")
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 1600 + K)
    Yi = poison((M, N), torch.int32)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi)
    np.testing.assert_array_equal(host(Yi), acc)
    del Yi
    Yh = poison((M, N), torch.float16)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh)
    assert f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y).max() <= 1
    del Yh
    if w8:
        W = wl.gen_weights(N, K, 1600 + K)
        ref8 = oracle.w8a8_pack(W)
        acc8, y8, _ = oracle.w8a8_gemm(host(X8), host(sx), ref8)
        pk8 = {"wq8": to_dev(ref8["wq8"]), "sw": to_dev(ref8["sw"]), "N": N, "K": K}
        Yi = poison((M, N), torch.int32)
        w4.gemm_w8a8(X8, sx, pk8, out_type=w4.OUT_I32, out=Yi)
        np.testing.assert_array_equal(host(Yi), acc8)
        Yh = poison((M, N), torch.float16)
        w4.gemm_w8a8(X8, sx, pk8, out_type=w4.OUT_F16, out=Yh)
        assert f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y8).max() <= 1


# 128-row plans that split K across two workgroups (or, when the extra X
# reads cost no more than the partials, an even number of them) run K parts
# instead: workgroups of 128 channels whose wave pairs take the two halves of
# the split's K range and add their int32 sums through LDS, with half the
# splits.  Every output element against the oracle, outputs and workspace
# poisoned (the same workspace twice):
#   128 x 2048 x 2816: 22 K-steps, two halves of 11 (odd: a padding step
#     each), no partials;
#   100 x 4096 x 2944: 23 K-steps, halves of 11 and 12 (the shorter runs one
#     X tile of zeros), ragged rows, group 64;
#   128 x 2048 x 4096: 32 K-steps, two splits of two parts of 8, reduced
#     from int32 partials;
#   128 x 512 x 4096: the same plan on two channel tiles, group 64;
#   128 x 3840 x 2048: 30 channel tiles (not a multiple of 8: the plain tile
#     order), no partials;
#   64 x 1024 x 8960: eight splits stay (X read again would cost more than
#     the partials), K-steps 8 or 9 per split;
#   128 x 2048 x 2560: halves of 10 K-steps.
# The W8A8 comparison runs the same plans.
_KPARTS = [(128, 2048, 2816, 128, True), (100, 4096, 2944, 64, True),
           (128, 2048, 4096, 128, True), (128, 512, 4096, 64, False),
           (128, 3840, 2048, 128, False), (64, 1024, 8960, 128, True),
           (128, 2048, 2560, 64, True)]


@pytest.mark.parametrize("M,N,K,g,w8", _KPARTS)
def test_k_parts_every_element(M, N, K, g, w8):
    say(f"K parts in the workgroup, every element: M={M} N={N} K={K} g={g}")
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 1800 + K)
    ws = poison((max(w4.workspace_size(M, N, K), 16),), torch.uint8)
    for _ in range(2):
        Yi = poison((M, N), torch.int32)
        w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi, workspace=ws)
        np.testing.assert_array_equal(host(Yi), acc)
        Yh = poison((M, N), torch.float16)
        w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh, workspace=ws)
        assert f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y).max() <= 1
    if w8:
        W = wl.gen_weights(N, K, 1800 + K)
        ref8 = oracle.w8a8_pack(W)
        acc8, y8, _ = oracle.w8a8_gemm(host(X8), host(sx), ref8)
        pk8 = {"wq8": to_dev(ref8["wq8"]), "sw": to_dev(ref8["sw"]), "N": N, "K": K}
        Yi = poison((M, N), torch.int32)
        w4.gemm_w8a8(X8, sx, pk8, out_type=w4.OUT_I32, out=Yi, workspace=ws)
        np.testing.assert_array_equal(host(Yi), acc8)
        Yh = poison((M, N), torch.float16)
        w4.gemm_w8a8(X8, sx, pk8, out_type=w4.OUT_F16, out=Yh, workspace=ws)
        assert f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y8).max() <= 1


def test_stream_params_from_global():
    """The streamed kernel reads the group parameters from global memory
    (byte loads per tile) when the parameter panels and X slots exceed its
    LDS budget: 20 x 4096 x 28672 with g = 64 runs two row blocks per
    workgroup, one tile, eight K-splitting waves, parameters not in LDS."""
    M, N, K, g = 20, 4096, 28672, 64
    say(f"streamed kernel, parameters from global memory: M={M} N={N} K={K} g={g}")
    X8, sx, pk, acc, y = _small_problem(M, N, K, g, 1701)
    Yi = poison((M, N), torch.int32)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi)
    np.testing.assert_array_equal(host(Yi), acc)
    Yh = poison((M, N), torch.float16)
    w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh)
    assert f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16), y).max() <= 1


def test_128_row_tiles_long_k():
    """128-row plans with more than 64 K-steps per workgroup run the
    32 x 32 x 32 tile kernel (1000 x 8192 x 8320: 256 tiles, no split, 65
    K-steps, ragged last row tile): sampled rows, int32 bit-exact and fp16
    within 1 ulp, for W4A8 and W8A8."""
    M, N, K, g = 1000, 8192, 8320, 64
    assert w4.workspace_size(M, N, K) == 0
    say(f"128-row tiles, long K: M={M} N={N} K={K} g={g}")
    rows = np.unique(np.concatenate([[0, 127, 128, 895, 896, M - 1],
                                     np.random.default_rng(19).choice(M, 10, replace=False)]))
    W = wl.gen_weights(N, K, 1501)
    X = wl.gen_activations(M, K, 1502, 1503)
    ref = oracle.w4a8_pack(W, g)
    X8, sx = oracle.quant_sym_rows(X, 127)
    pk = {"wq": to_dev(ref["wq"]), "s_u8": to_dev(ref["s_panels"]),
          "a_u8": to_dev(ref["a_panels"]), "sw": to_dev(ref["sw"]), "N": N, "K": K, "group": g}
    Yi = poison((M, N), torch.int32)
    w4.gemm(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_I32, out=Yi)
    Yh = poison((M, N), torch.float16)
    w4.gemm(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F16, out=Yh)
    acc, y, _ = oracle.w4a8_gemm(X8[rows], sx[rows], ref, g)
    np.testing.assert_array_equal(host(Yi)[rows], acc)
    assert f16_ulp_diff(host(Yh.view(torch.int16)).view(np.uint16)[rows], y).max() <= 1
    ref8 = oracle.w8a8_pack(W)
    pk8 = {"wq8": to_dev(ref8["wq8"]), "sw": to_dev(ref8["sw"]), "N": N, "K": K}
    Yi = poison((M, N), torch.int32)
    w4.gemm_w8a8(to_dev(X8), to_dev(sx), pk8, out_type=w4.OUT_I32, out=Yi)
    acc8, _, _ = oracle.w8a8_gemm(X8[rows], sx[rows], ref8)
    np.testing.assert_array_equal(host(Yi)[rows], acc8)


def test_fp8g_end_to_end_device_pack():
    """Device pack then device GEMM equals oracle pack then device GEMM bit
    for bit (the packed inputs are identical, so the outputs must be)."""
    M, N, K, g = 200, 512, 1024, 128
    W = _fp8g_weights(N, K, g, 901)
    X = wl.gen_activations(M, K, 902, 903)
    X8, sx = oracle.quant_rows_e4m3(X)
    ref_pk = oracle.w4fp8g_pack(W, g)
    a = w4.gemm_fp8g(to_dev(X8), to_dev(sx), w4.pack_fp8g(to_dev(W), group=g),
                     out_type=w4.OUT_F32)
    b = w4.gemm_fp8g(to_dev(X8), to_dev(sx), _fp8g_device(ref_pk, N, K, g), out_type=w4.OUT_F32)
    np.testing.assert_array_equal(host(a).view(np.uint32), host(b).view(np.uint32))


# ---------------------------------------------- largest accepted sizes ----
def test_largest_activation_extent():
    """M * K just below 2^31, the largest activation extent the entry points
    accept: the kernels address X with 32-bit buffer offsets, so the last
    rows sit at offsets near the top of that range.  16256 x 256 x 131072
    runs the 32 x 32 tile kernel with two K splits (int32 partials in the
    workspace); an explicit split factor runs the streamed kernel over all
    1016 row blocks.  Sampled rows, the first and the last among them, match
    the oracle: int32 exactly, fp16 within 1 ulp."""
    M, N, K, g = 16256, 256, 131072, 128
    assert M * K < (1 << 31) <= (M + 128) * K  # one more 128-row tile would not fit
    plan = w4.gemm_plan(M, N, K)
    assert (plan["kernel"], plan["splits"]) == ("tile32", 2), plan
    say(f"largest activation extent M={M} N={N} K={K} plan={plan}")
    W = wl.gen_weights(N, K, 4242)
    pk_ref = oracle.w4a8_pack(W, g)
    pk = {"wq": to_dev(pk_ref["wq"]), "s_u8": to_dev(pk_ref["s_panels"]),
          "a_u8": to_dev(pk_ref["a_panels"]), "sw": to_dev(pk_ref["sw"]),
          "N": N, "K": K, "group": g}
    del W
    rng = np.random.default_rng(4243)
    X8 = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    sx = rng.uniform(1e-3, 2e-2, size=M).astype(np.float32)
    rows = np.array([0, 1, 2, M // 2, M - 129, M - 17, M - 2, M - 1])
    acc, y, _ = oracle.w4a8_gemm(X8[rows], sx[rows], pk_ref, g)
    Xd, sxd = to_dev(X8), to_dev(sx)
    del X8
    for sk in (0, 1):
        say(f"  splitk={sk}")
        Yi = poison((M, N), torch.int32)
        w4.gemm(Xd, sxd, pk, out_type=w4.OUT_I32, splitk=sk, out=Yi)
        np.testing.assert_array_equal(host(Yi[to_dev(rows)]), acc)
        del Yi
        Yh = poison((M, N), torch.float16)
        w4.gemm(Xd, sxd, pk, out_type=w4.OUT_F16, splitk=sk, out=Yh)
        d = f16_ulp_diff(host(Yh[to_dev(rows)].view(torch.int16)).view(np.uint16), y)
        assert d.max() <= 1
        del Yh
    del Xd


def test_largest_weight_extent():
    """N * K just below 2^32 codes, the largest weight extent the entry points
    accept: 2 GiB of packed codes, addressed with 32-bit buffer offsets.
    Random codes and valid group parameters (s in 1..16, a <= 255 - 15 s, so
    q*s + a stays a byte), built directly in the packed layout; the oracle
    decodes sampled channels, the last ones among them, from their own 16-channel
    slabs.  M = 16 runs the streamed kernel, M = 128 the 128-row tile kernel;
    the FP8 kernels read the same codes as sign-magnitude INT4 (integer
    activations, unit scales: exact float32 sums)."""
    N, K, g = 524032, 8192, 128
    assert N * K < (1 << 32) <= (N + 256) * K  # one more 256-channel tile would not fit
    KT, G = K // 128, K // g
    rng = np.random.default_rng(4244)
    wq = rng.integers(0, 256, size=N * K // 2, dtype=np.uint8)
    s_rm = rng.integers(1, 17, size=(N, G), dtype=np.uint8)
    a_rm = (1 + rng.integers(0, 1 << 16, size=(N, G)) % (255 - 15 * s_rm.astype(np.int64))
            ).astype(np.uint8)
    sw = rng.uniform(1e-4, 1e-3, size=N).astype(np.float32)
    chans = np.array([0, 1, 255, N // 2 + 7, N - 257, N - 17, N - 2, N - 1])

    def codes_of(n):  # the 16-channel slab of channel n holds all its K-tiles
        slab = wq[(n // 16) * KT * 1024:(n // 16 + 1) * KT * 1024]
        return oracle.unpack_nibbles(slab, 16, K)[n % 16]

    codes = np.stack([codes_of(n) for n in chans])
    sub = {"codes": codes, "s_u8": s_rm[chans], "a_u8": a_rm[chans], "sw": sw[chans]}
    pk = {"wq": to_dev(wq), "s_u8": to_dev(oracle.params_to_panels(s_rm)),
          "a_u8": to_dev(oracle.params_to_panels(a_rm)), "sw": to_dev(sw),
          "N": N, "K": K, "group": g}
    del wq
    cidx = to_dev(chans)
    for M in (16, 128):
        plan = w4.gemm_plan(M, N, K)
        say(f"largest weight extent M={M} N={N} K={K} plan={plan}")
        X8 = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
        sx = rng.uniform(1e-3, 2e-2, size=M).astype(np.float32)
        acc, y, _ = oracle.w4a8_gemm(X8, sx, sub, g)
        Yi = poison((M, N), torch.int32)
        w4.gemm(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_I32, out=Yi)
        np.testing.assert_array_equal(host(Yi[:, cidx]), acc)
        del Yi
        Yh = poison((M, N), torch.float16)
        w4.gemm(to_dev(X8), to_dev(sx), pk, out_type=w4.OUT_F16, out=Yh)
        d = f16_ulp_diff(host(Yh[:, cidx].view(torch.int16)).view(np.uint16), y)
        assert d.max() <= 1
        del Yh
        # FP8 kernels: integer activations in [-16, 16] (exact in e4m3)
        Xi = rng.integers(-16, 17, size=(M, K)).astype(np.float64)
        Xe = oracle.e4m3_encode(Xi)
        q = oracle.int4_sm_values(codes).astype(np.int64)
        exact = (Xi.astype(np.int64) @ q.T).astype(np.float32)
        pk8 = {"wq": pk["wq"], "sw": to_dev(np.ones(N, np.float32)), "N": N, "K": K}
        Yf = poison((M, N), torch.float32)
        w4.gemm_fp8(to_dev(Xe), to_dev(np.ones(M, np.float32)), pk8, out_type=w4.OUT_F32,
                    out=Yf)
        np.testing.assert_array_equal(host(Yf[:, cidx]), exact)
        del Yf


# ------------------------------------------- Llama-shaped workloads --------
_FULL = [(c, sh) for c in (wl.LLAMA7B_DECODE, wl.LLAMA7B_PREFILL, wl.LLAMA70B_SWEEP)
         for sh in wl.CONFIGS[c].shapes]

_packed_cache = {}


def _device_packed(cfg, sh):
    key = (cfg, sh.N, sh.K, sh.group)
    if key not in _packed_cache:
        _packed_cache.clear()
        pair = wl.nk_pairs(cfg).index((sh.N, sh.K))
        W = wl.gen_weights(sh.N, sh.K, wl.seed_w(cfg, pair))
        pk = w4.pack(to_dev(W), group=sh.group)
        torch.cuda.synchronize()
        _packed_cache[key] = (W, pk)
    return _packed_cache[key]


@pytest.mark.parametrize("cfg,sh", _FULL, ids=[s.name for _, s in _FULL])
def test_llama_shapes_sampled(cfg, sh):
    say(f"full-size {sh.name}: M={sh.M} N={sh.N} K={sh.K} g={sh.group}")
    W, pk = _device_packed(cfg, sh)
    X = wl.gen_activations(sh.M, sh.K, wl.seed_x(cfg, sh.M), wl.seed_outliers(cfg))
    Xq, sx = w4.quant_act(to_dev(X))
    Yh = poison((sh.M, sh.N), torch.float16)
    w4.gemm(Xq, sx, pk, out_type=w4.OUT_F16, out=Yh)
    Yi = poison((sh.M, sh.N), torch.int32)
    w4.gemm(Xq, sx, pk, out_type=w4.OUT_I32, out=Yi)
    torch.cuda.synchronize()
    rng = np.random.default_rng(sh.M * 7 + sh.N)
    nsel = np.sort(rng.choice(sh.N, 48, replace=False))
    msel = np.arange(sh.M) if sh.M <= 16 else np.sort(rng.choice(sh.M, 12, replace=False))
    # weights: oracle packing of the sampled channels vs the device's bytes
    ref = oracle.w4a8_pack(W[nsel], sh.group)  # row sample: panel order not used
    codes_dev = oracle.unpack_nibbles(host(pk["wq"]), sh.N, sh.K)[nsel]
    np.testing.assert_array_equal(codes_dev, ref["codes"])
    groups = sh.K // sh.group
    s_dev = oracle.params_from_panels(host(pk["s_u8"]), sh.N, groups)
    a_dev = oracle.params_from_panels(host(pk["a_u8"]), sh.N, groups)
    np.testing.assert_array_equal(s_dev[nsel], ref["s_u8"])
    np.testing.assert_array_equal(a_dev[nsel], ref["a_u8"])
    np.testing.assert_array_equal(host(pk["sw"])[nsel], ref["sw"])
    # activations: sampled tokens
    X8, sx8 = oracle.quant_sym_rows(X[msel], 127)
    np.testing.assert_array_equal(host(Xq)[msel], X8)
    np.testing.assert_array_equal(host(sx)[msel], sx8)
    # GEMM on the sample
    acc, y, _ = oracle.w4a8_gemm(X8, sx8, ref, sh.group)
    np.testing.assert_array_equal(host(Yi)[np.ix_(msel, nsel)], acc)
    yh = host(Yh.view(torch.int16)).view(np.uint16)[np.ix_(msel, nsel)]
    assert f16_ulp_diff(yh, y).max() <= 1


def test_fp8_variant_full_size_sampled():
    sh = wl.CONFIGS[wl.FP8_VARIANT].shapes[0]
    say(f"full-size {sh.name}: M={sh.M} N={sh.N} K={sh.K}")
    W = wl.gen_weights(sh.N, sh.K, wl.seed_w(wl.FP8_VARIANT))
    X = wl.gen_activations(sh.M, sh.K, wl.seed_x(wl.FP8_VARIANT), wl.seed_outliers(wl.FP8_VARIANT))
    pk = w4.pack(to_dev(W), mode=w4.PACK_INT4_SYM)
    Xq, sx = w4.quant_act_fp8(to_dev(X))
    Yf = w4.gemm_fp8(Xq, sx, pk, out_type=w4.OUT_F32)
    Yb = w4.gemm_fp8(Xq, sx, pk, out_type=w4.OUT_BF16)
    rng = np.random.default_rng(4)
    nsel = np.sort(rng.choice(sh.N, 64, replace=False))
    msel = np.sort(rng.choice(sh.M, 24, replace=False))
    ref_pk = oracle.w4fp8_pack(W[nsel])
    codes_dev = oracle.unpack_nibbles(host(pk["wq"]), sh.N, sh.K)[nsel]
    np.testing.assert_array_equal(codes_dev, ref_pk["codes"])
    X8, sx8 = oracle.quant_rows_e4m3(X[msel])
    np.testing.assert_array_equal(host(Xq)[msel], X8)
    ref, _ = oracle.w4fp8_ref(X8, sx8, ref_pk["q"], ref_pk["sw"])
    bound = _fp8_bound(X8, sx8, ref_pk["q"], ref_pk["sw"])
    _check_fp8_outputs(host(Yf)[np.ix_(msel, nsel)], bf16_bits_of(Yb)[np.ix_(msel, nsel)],
                       ref, bound)
    err = rel_fro(host(Yf)[np.ix_(msel, nsel)], ref)
    gv = (bf16_bits_of(Yb)[np.ix_(msel, nsel)].astype(np.uint32) << 16).view(np.float32)
    wv = (oracle.round_bf16(ref).astype(np.uint32) << 16).view(np.float32)
    err_b = rel_fro(gv, wv)
    say(f"  f32 rel fro {err:.3e}  bf16 vs bf16(ref) {err_b:.3e}  bf16 vs ref {rel_fro(gv, ref):.3e}")
    assert err <= 1e-3 and err_b <= 1e-3
