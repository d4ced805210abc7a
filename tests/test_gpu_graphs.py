"""The GEMM entry points under HIP graph capture (serving loops replay a
captured decode step instead of launching kernel by kernel).

The library allocates nothing and issues no memset or copy, so a captured
call is just its kernel launches.  Each graph is replayed several times
with eager work in between (the outputs are overwritten eagerly before
every replay), and every replay must reproduce the eager result bit for
bit.  The last test runs calls on several streams at once: the entry points
share no state, so overlapping calls give the serial results.
"""
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


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _w4a8_case(M, N, K, g, seed):
    W = wl.gen_weights(N, K, seed)
    X = wl.gen_activations(M, K, seed + 1, seed + 2)
    pk_ref = oracle.w4a8_pack(W, g)
    X8, sx = oracle.quant_sym_rows(X, 127)
    pk = {"wq": to_dev(pk_ref["wq"]), "s_u8": to_dev(pk_ref["s_panels"]),
          "a_u8": to_dev(pk_ref["a_panels"]), "sw": to_dev(pk_ref["sw"]),
          "N": N, "K": K, "group": g}
    return to_dev(X8), to_dev(sx), pk


def _replay_and_check(calls, outs, replays=3):
    """calls: list of zero-argument functions writing into `outs`."""
    for fn in calls:  # warm-up (and eager reference)
        fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in calls:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for fn in calls:
            fn()
    for r in range(replays):
        for o in outs:  # eager work between replays
            o.view(torch.uint8).fill_(0xA5 + r)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"replay {r}"


def test_graph_w4a8_decode_and_tiles():
    """A decode-shaped call (streamed kernel), an unsplit tile call and a
    split-K tile call (workspace partials + ordered reduction) in one graph."""
    cases = [(16, 1024, 2048, 128, 11), (512, 512, 1024, 64, 12), (128, 256, 4096, 128, 13)]
    calls, outs = [], []
    for (M, N, K, g, seed) in cases:
        X8, sx, pk = _w4a8_case(M, N, K, g, seed)
        need = w4.workspace_size(M, N, K)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
        Yh = torch.empty((M, N), dtype=torch.float16, device=DEV)
        Yi = torch.empty((M, N), dtype=torch.int32, device=DEV)
        calls.append(lambda X8=X8, sx=sx, pk=pk, ws=ws, Yh=Yh:
                     w4.gemm(X8, sx, pk, out_type=w4.OUT_F16, out=Yh, workspace=ws))
        calls.append(lambda X8=X8, sx=sx, pk=pk, ws=ws, Yi=Yi:
                     w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Yi, workspace=ws))
        outs += [Yh, Yi]
    assert w4.workspace_size(128, 256, 4096) > 0  # the split-K case really splits
    _replay_and_check(calls, outs)


def test_graph_quant_act_then_gemm():
    """The whole decode step as a serving loop captures it: per-token
    quantisation of fp16 activations, then the GEMM."""
    M, N, K, g = 16, 512, 1024, 64
    _, _, pk = _w4a8_case(M, N, K, g, 21)
    Xh = torch.from_numpy(wl.gen_activations(M, K, 22, 23)).to(DEV).to(torch.float16)
    Xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    sx = torch.empty(M, dtype=torch.float32, device=DEV)
    Y = torch.empty((M, N), dtype=torch.float16, device=DEV)

    def step():
        w4.quant_act(Xh, out=(Xq, sx))
        w4.gemm(Xq, sx, pk, out=Y)
    _replay_and_check([step], [Xq, sx, Y])


def test_graph_fp8_and_grouped():
    """FP8 (tile kernel, folded format through the streamed kernel) and the
    grouped mixture-of-experts GEMM with device-side offsets."""
    M, N, K = 128, 256, 1024
    W = wl.gen_weights(N, K, 31)
    X = wl.gen_activations(M, K, 32, 33)
    X8, sx8 = oracle.quant_rows_e4m3(X)
    X8, sx8 = to_dev(X8), to_dev(sx8)
    pk8 = w4.pack(to_dev(W), mode=w4.PACK_INT4_SYM)
    pkg = w4.pack_fp8g(to_dev(W), group=128)
    Yb = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    Yg = torch.empty((16, N), dtype=torch.float32, device=DEV)
    E, Ng, Kg, g = 4, 256, 512, 64
    Ws = torch.from_numpy(np.stack([wl.gen_weights(Ng, Kg, 40 + e) for e in range(E)])).to(DEV)
    pke = w4.pack_experts(Ws, group=g)
    counts = [5, 0, 70, 1]
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device=DEV)
    Mg = int(sum(counts))
    Xe = torch.from_numpy(wl.gen_activations(Mg, Kg, 44, 45)).to(DEV)
    Xqe, sxe = w4.quant_act(Xe)
    Ye = torch.empty((Mg, Ng), dtype=torch.float16, device=DEV)
    calls = [lambda: w4.gemm_fp8(X8, sx8, pk8, out=Yb),
             lambda: w4.gemm_fp8g(X8[:16], sx8[:16], pkg, out_type=w4.OUT_F32, out=Yg),
             lambda: w4.gemm_grouped(Xqe, sxe, offs, pke, max(counts), out=Ye)]
    _replay_and_check(calls, [Yb, Yg, Ye])


def test_graph_row_blocks_and_quant():
    """Streamed calls with two and four 16-row blocks per workgroup, and both
    activation quantisers at both thread counts per row (fewer / more rows
    than CUs)."""
    calls, outs = [], []
    for (M, N, K, g, seed) in ((24, 8192, 1024, 64, 51), (40, 8192, 1024, 128, 52)):
        X8, sx, pk = _w4a8_case(M, N, K, g, seed)
        Yh = torch.empty((M, N), dtype=torch.float16, device=DEV)
        calls.append(lambda X8=X8, sx=sx, pk=pk, Yh=Yh: w4.gemm(X8, sx, pk, out=Yh))
        outs.append(Yh)
    for (M, K, seed) in ((16, 4096, 53), (300, 2048, 54)):
        Xh = torch.from_numpy(wl.gen_activations(M, K, seed, seed + 1)).to(DEV).to(torch.float16)
        q8 = torch.empty((M, K), dtype=torch.int8, device=DEV)
        s8 = torch.empty(M, dtype=torch.float32, device=DEV)
        qe = torch.empty((M, K), dtype=torch.uint8, device=DEV)
        se = torch.empty(M, dtype=torch.float32, device=DEV)
        calls.append(lambda Xh=Xh, q8=q8, s8=s8: w4.quant_act(Xh, out=(q8, s8)))
        calls.append(lambda Xh=Xh, qe=qe, se=se: w4.quant_act_fp8(Xh, out=(qe, se)))
        outs += [q8, s8, qe, se]
    _replay_and_check(calls, outs)


def test_concurrent_streams():
    """Calls share no state: several GEMMs (streamed, tile, split-K with a
    workspace each, and the FP8 tile kernel) enqueued on four streams, so
    their kernels overlap on the GPU, give the same bits as the same calls
    run one after another on one stream."""
    cases = [(16, 1024, 2048, 128, 31), (512, 512, 1024, 64, 32), (128, 256, 4096, 128, 33),
             (200, 1024, 8192, 128, 34)]
    calls, outs = [], []
    for (M, N, K, g, seed) in cases:
        X8, sx, pk = _w4a8_case(M, N, K, g, seed)
        ws = torch.empty(max(w4.workspace_size(M, N, K), 16), dtype=torch.uint8, device=DEV)
        Y = torch.empty((M, N), dtype=torch.int32, device=DEV)
        calls.append(lambda X8=X8, sx=sx, pk=pk, ws=ws, Y=Y:
                     w4.gemm(X8, sx, pk, out_type=w4.OUT_I32, out=Y, workspace=ws))
        outs.append(Y)
    M, N, K = 300, 512, 2048
    rng = np.random.default_rng(35)
    q = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    X8f = oracle.e4m3_encode(rng.integers(-16, 17, size=(M, K)).astype(np.float64))
    pk8 = {"wq": to_dev(oracle.pack_nibbles(oracle.int4_sm_codes(q))),
           "sw": to_dev(np.ones(N, np.float32)), "N": N, "K": K}
    X8d, ones = to_dev(X8f), to_dev(np.ones(M, np.float32))
    Yf = torch.empty((M, N), dtype=torch.float32, device=DEV)
    calls.append(lambda: w4.gemm_fp8(X8d, ones, pk8, out_type=w4.OUT_F32, out=Yf))
    outs.append(Yf)
    assert w4.workspace_size(128, 256, 4096) > 0 and w4.workspace_size(200, 1024, 8192) > 0
    for fn in calls:  # one after another on the current stream
        fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    streams = [torch.cuda.Stream() for _ in range(4)]
    for r in range(3):
        for o in outs:
            o.view(torch.uint8).fill_(0x5A + r)
        torch.cuda.synchronize()
        for i, fn in enumerate(calls):
            with torch.cuda.stream(streams[i % 4]):
                fn()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"round {r}"
