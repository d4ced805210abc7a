"""The kernel plan w4a8_gemm takes, through w4a8_gemm_plan (host logic, no
GPU): the benchmark's slots, the Llama-2-7B rows, and the shapes whose GPU
parity tests are chosen to reach a particular plan, so that a change of the
plan rule cannot leave those tests exercising something else unnoticed."""
import ctypes

import pytest

import w4a8_quantized_gemm_amd as w4

T16, T32, ST = "tile16", "tile32", "stream"


def plan(M, N, K, splitk=0):
    p = w4.gemm_plan(M, N, K, splitk)
    return (p["kernel"], p["tile_rows"], p["tile_channels"], p["splits"], p["k_parts"])


# Llama-2-70B MLP shapes at the benchmark's M, and the 7B rows
BENCH = {
    (4096, 28672, 8192): (T16, 256, 256, 1, 1),
    (4096, 8192, 28672): (T16, 256, 256, 1, 1),
    (1024, 28672, 8192): (T16, 128, 256, 1, 1),   # two workgroups per CU
    (1024, 8192, 28672): (T32, 128, 256, 1, 1),   # long K, one per CU
    (128, 28672, 8192): (T16, 128, 128, 1, 2),    # K parts, no partials
    (128, 8192, 28672): (T16, 128, 256, 8, 1),    # eight splits
    (16, 28672, 8192): (ST, 16, 64, 1, 4),
    (16, 8192, 28672): (ST, 16, 32, 1, 8),
    (1, 28672, 8192): (ST, 16, 64, 1, 4),
    (1, 8192, 28672): (ST, 16, 32, 1, 8),
    (1, 4096, 4096): (ST, 16, 16, 1, 8),
    (16, 4096, 4096): (ST, 16, 16, 1, 8),
    (2048, 11008, 4096): (T16, 128, 256, 1, 1),
    (2048, 4096, 11008): (T32, 128, 256, 1, 1),
}

# shapes of the GPU parity tests, with the plan their docstrings and
# comments name
PARITY = {
    # K parts: halves of 11 / 11 and 12 / two splits of two parts / 30 tiles
    (128, 2048, 2816): (T16, 128, 128, 1, 2),
    (100, 4096, 2944): (T16, 128, 128, 1, 2),
    (128, 2048, 4096): (T16, 128, 128, 2, 2),
    (128, 512, 4096): (T16, 128, 128, 2, 2),
    (128, 3840, 2048): (T16, 128, 128, 1, 2),
    (128, 2048, 2560): (T16, 128, 128, 1, 2),
    (64, 1024, 8960): (T16, 128, 256, 8, 1),      # eight splits stay
    (100, 256, 2048): (T16, 128, 128, 1, 2),
    # the 256-row plan of the 16 x 16 kernel
    (4096, 16384, 256): (T16, 256, 256, 1, 1),
    (4096, 16384, 384): (T16, 256, 256, 1, 1),
    (4000, 4096, 8320): (T16, 256, 256, 1, 1),
    (4096, 4096, 8448): (T16, 256, 256, 1, 1),
    (4000, 4864, 8448): (T16, 256, 256, 1, 1),
    (4000, 8192, 8320): (T16, 256, 256, 1, 1),
    # long-K 128-row tiles on the 32 x 32 kernel
    (1000, 8192, 8320): (T32, 128, 256, 1, 1),
    # any integer split count
    (600, 4352, 3072): (T16, 128, 256, 3, 1),
    (640, 2048, 6272): (T16, 128, 256, 6, 1),
    (100, 6912, 9216): (T16, 128, 256, 9, 1),
    (128, 6144, 10368): (T16, 128, 256, 10, 1),
    (128, 4352, 15360): (T16, 128, 256, 15, 1),
    (100, 256, 16384): (T16, 128, 256, 16, 1),
    # streamed: parameters from global memory (two row blocks, one tile)
    (20, 4096, 28672): (ST, 32, 16, 1, 8),
    (20, 2048, 65536): (ST, 16, 16, 1, 8),        # one row block, g = 128
    # a single K-step on either kernel
    (16, 128, 128): (ST, 16, 16, 1, 1),
    (128, 512, 128): (T16, 128, 256, 1, 1),
}


@pytest.mark.parametrize("shape,want", list(BENCH.items()) + list(PARITY.items()),
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v[0], int) else None)
def test_plan(shape, want):
    assert plan(*shape) == want


def test_splitk_forces_the_streamed_kernel():
    # an explicit split factor runs the streamed kernel, one tile per
    # workgroup, with that many K-splitting waves
    for M, N, K, s in [(4096, 28672, 8192, 4), (128, 8192, 28672, 16), (16, 4096, 4096, 1)]:
        kernel, _, chans, splits, parts = plan(M, N, K, splitk=s)
        assert (kernel, chans, splits, parts) == (ST, 16, 1, s)


def test_workspace_matches_the_splits():
    # w4a8_workspace_size covers every entry point: int32 partials for the
    # split count of the plan without K parts
    assert w4.workspace_size(128, 8192, 28672) == 8 * 128 * 8192 * 4
    assert w4.workspace_size(4096, 28672, 8192) == 0


def test_empty_problem_plan():
    assert plan(0, 4096, 4096)[0] == ST
    assert plan(128, 0, 4096)[0] == ST


def test_plan_errors():
    out = [ctypes.c_int(0) for _ in range(5)]
    ptrs = [ctypes.addressof(v) for v in out]
    assert w4.lib.w4a8_gemm_plan(16, 4096, 4096, 0, None, *ptrs[1:]) == 1     # NULL
    assert w4.lib.w4a8_gemm_plan(16, 100, 4096, 0, *ptrs) == 2                # N % 64
    assert w4.lib.w4a8_gemm_plan(16, 4096, 4000, 0, *ptrs) == 2               # K % 128
    assert w4.lib.w4a8_gemm_plan(-1, 4096, 4096, 0, *ptrs) == 2
    assert w4.lib.w4a8_gemm_plan(16, 4096, 4096, 3, *ptrs) == 2               # splitk
