"""w4a8_gemm_noalloc against w4a8_gemm, through the C ABI.

The no-allocation entry point runs the same kernels with the library's
static device scratch as the split-K workspace, so its outputs must equal
w4a8_gemm's bit for bit (int32 accumulators and fp16 outputs).  Two calls in
a row, the second on a smaller problem, check that what the first call
leaves in the shared scratch does not leak into the second; both are also
checked against the CPU oracle (int32 exact, fp16 within 1 ulp).
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a8_quantized_gemm_amd as w4  # noqa: E402

DEV = "cuda:0"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _problem(M, N, K, g, seed):
    W = wl.gen_weights(N, K, seed)
    X = wl.gen_activations(M, K, seed + 1, seed + 2)
    ref = oracle.w4a8_pack(W, g)
    X8, sx = oracle.quant_sym_rows(X, 127)
    acc, y, _ = oracle.w4a8_gemm(X8, sx, ref, g)
    pk = {"wq": _dev(ref["wq"]), "s_u8": _dev(ref["s_panels"]), "a_u8": _dev(ref["a_panels"]),
          "sw": _dev(ref["sw"]), "N": N, "K": K, "group": g}
    return _dev(X8), _dev(sx), pk, acc, y


def _noalloc(X, sx, pk, Y, out_type):
    M, K = X.shape
    st = w4.lib.w4a8_gemm_noalloc(X.data_ptr(), sx.data_ptr(), pk["wq"].data_ptr(),
                                  pk["s_u8"].data_ptr(), pk["a_u8"].data_ptr(),
                                  pk["sw"].data_ptr(), Y.data_ptr(), out_type, M, pk["N"], K,
                                  pk["group"], 0,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, w4.lib.w4a8_status_str(st)


def _poison(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(0xAB)
    return t


def _ulp(a, b):
    def o(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u & 0x7FFF)
    return np.abs(o(a) - o(b))


# split-K shapes (the scratch holds their partials; the second is smaller
# and leaves most of what the first wrote in place), then a streamed-kernel
# shape that uses no scratch
CASES = [(128, 4096, 8192, 128), (100, 2048, 4096, 64), (16, 1024, 2048, 64)]


def test_noalloc_matches_gemm_two_calls():
    for i, (M, N, K, g) in enumerate(CASES):
        print(f"noalloc call {i}: M={M} N={N} K={K} g={g} "
              f"workspace={w4.workspace_size(M, N, K)}", flush=True)
        assert w4.workspace_size(M, N, K) <= (32 << 20)
        X8, sx, pk, acc, y = _problem(M, N, K, g, 4100 + i)
        for out_type, dt in ((w4.OUT_I32, torch.int32), (w4.OUT_F16, torch.float16)):
            Ya = _poison((M, N), dt)
            w4.gemm(X8, sx, pk, out_type=out_type, out=Ya)
            Yb = _poison((M, N), dt)
            _noalloc(X8, sx, pk, Yb, out_type)
            torch.cuda.synchronize()
            a, b = Ya.cpu().numpy(), Yb.cpu().numpy()
            np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8))
            if out_type == w4.OUT_I32:
                np.testing.assert_array_equal(b, acc)
            else:
                assert _ulp(b.view(np.uint16), y).max() <= 1


def test_noalloc_in_captured_graph():
    """The callers this entry point is for capture it in a HIP graph: three
    split-K calls of different shapes sharing the static scratch, captured
    once and replayed three times with eager work in between; every replay
    equals eager w4a8_gemm bit for bit."""
    cases = [(128, 4096, 8192, 128), (100, 2048, 4096, 64), (192, 1024, 8192, 128)]
    probs = [_problem(M, N, K, g, 4200 + i) for i, (M, N, K, g) in enumerate(cases)]
    outs = [_poison((M, N), torch.float16) for (M, N, K, g) in cases]
    want = []
    for (X8, sx, pk, acc, y), (M, N, K, g) in zip(probs, cases):
        assert w4.workspace_size(M, N, K) > 0
        ref = _poison((M, N), torch.float16)
        w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=ref)
        want.append(ref)
    for (X8, sx, pk, _, _), Y in zip(probs, outs):  # first call on the device: eager
        _noalloc(X8, sx, pk, Y, w4.OUT_F16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for (X8, sx, pk, _, _), Y in zip(probs, outs):
                _noalloc(X8, sx, pk, Y, w4.OUT_F16)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for Y in outs:
            Y.view(torch.uint8).fill_(0xAB)
        X8, sx, pk, _, _ = probs[0]
        w4.gemm(X8, sx, pk, out_type=w4.OUT_I32)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for Y, ref in zip(outs, want):
            np.testing.assert_array_equal(Y.cpu().numpy().view(np.uint16),
                                          ref.cpu().numpy().view(np.uint16))
