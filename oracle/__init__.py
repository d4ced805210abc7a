"""CPU oracle for the W4A8 / W4FP8 GEMM paths (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP
library ``w4a8_quantized_gemm_amd``: the arithmetic lives in ``oracle.c``
(plain C loops, compiled with gcc), this file only marshals numpy arrays.

Every step cites the passage it follows; see ``oracle.c`` for the step
definitions and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add may change a rounding step.
CFLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc; returns the path."""
    if force or not os.path.exists(_LIB) or \
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int64
_F = ctypes.c_float


def _declare(L):
    sig = {
        "orc_quant_sym_rows": ([_P, _I, _I, _F, _P, _P], None),
        "orc_lqq_encode": ([_P, _I, _I, _I, _P, _P, _P, _P], None),
        "orc_lqq_decode": ([_P, _P, _P, _I, _I, _I, _P], ctypes.c_int64),
        "orc_pack_nibbles": ([_P, _I, _I, _P], None),
        "orc_unpack_nibbles": ([_P, _I, _I, _P], None),
        "orc_params_to_panels": ([_P, _I, _I, _P], None),
        "orc_params_from_panels": ([_P, _I, _I, _P], None),
        "orc_gemm_i32": ([_P, _P, _I, _I, _I, _P], None),
        "orc_round_f16": ([_P, _I, _P], None),
        "orc_round_bf16": ([_P, _I, _P], None),
        "orc_epilogue_f16": ([_P, _P, _P, _I, _I, _P, _P], None),
        "orc_e4m3_decode": ([_P, _I, _P], None),
        "orc_e4m3_encode": ([_P, _I, _P], None),
        "orc_quant_rows_e4m3": ([_P, _I, _I, _P, _P], None),
        "orc_int4_sm_codes": ([_P, _I, _P], None),
        "orc_int4_sm_values": ([_P, _I, _P], None),
        "orc_w4fp8_ref": ([_P, _P, _P, _P, _I, _I, _I, _P, _P], None),
        "orc_w4fp8g_pack": ([_P, _I, _I, _I, _P, _P, _P, _P], None),
        "orc_w4fp8g_weights": ([_P, _P, _I, _I, _I, _P], None),
        "orc_w4fp8g_ref": ([_P, _P, _P, _F, _I, _I, _I, _P, _P], None),
        "orc_pack_w8": ([_P, _I, _I, _P], None),
        "orc_unpack_w8": ([_P, _I, _I, _P], None),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- steps ----

def quant_sym_rows(x, qmax: float):
    """Per-row symmetric quantisation: (int8 codes, float32 scales)."""
    x = _c(x, np.float32)
    R, C = x.shape
    q = np.empty((R, C), np.int8)
    s = np.empty(R, np.float32)
    lib().orc_quant_sym_rows(_p(x), R, C, float(qmax), _p(q), _p(s))
    return q, s


def lqq_encode(Q, g: int):
    """LiquidQuant second level: (codes [N][K] u8, s_u8, a_u8, n_saturated)."""
    Q = _c(Q, np.int8)
    N, K = Q.shape
    assert K % g == 0
    codes = np.empty((N, K), np.uint8)
    s = np.empty((N, K // g), np.uint8)
    a = np.empty((N, K // g), np.uint8)
    nsat = ctypes.c_int64(0)
    lib().orc_lqq_encode(_p(Q), N, K, g, _p(codes), _p(s), _p(a),
                         ctypes.addressof(nsat))
    return codes, s, a, int(nsat.value)


def lqq_decode(codes, s, a, g: int, check_carry: bool = True):
    """The identity (q*s + a) XOR 0x80 on bytes -> int8 [N][K]."""
    codes = _c(codes, np.uint8)
    s = _c(s, np.uint8)
    a = _c(a, np.uint8)
    N, K = codes.shape
    out = np.empty((N, K), np.int8)
    carries = lib().orc_lqq_decode(_p(codes), _p(s), _p(a), N, K, g, _p(out))
    if check_carry and carries:
        raise AssertionError(f"LQQ decode: {carries} UINT8 carries")
    return out


def pack_nibbles(codes):
    codes = _c(codes, np.uint8)
    N, K = codes.shape
    assert N % 16 == 0 and K % 128 == 0
    wq = np.empty(N * K // 2, np.uint8)
    lib().orc_pack_nibbles(_p(codes), N, K, _p(wq))
    return wq


def unpack_nibbles(wq, N: int, K: int):
    wq = _c(wq, np.uint8).reshape(-1)
    assert wq.size == N * K // 2
    codes = np.empty((N, K), np.uint8)
    lib().orc_unpack_nibbles(_p(wq), N, K, _p(codes))
    return codes


def params_to_panels(p):
    """Row-major [N][K/g] group parameters -> the library's panel order."""
    p = _c(p, np.uint8)
    N, groups = p.shape
    assert N % 64 == 0
    out = np.empty(N * groups, np.uint8)
    lib().orc_params_to_panels(_p(p), N, groups, _p(out))
    return out


def params_from_panels(panels, N: int, groups: int):
    """The library's panel order -> row-major [N][groups]."""
    panels = _c(panels, np.uint8).reshape(-1)
    assert panels.size == N * groups and N % 64 == 0
    out = np.empty((N, groups), np.uint8)
    lib().orc_params_from_panels(_p(panels), N, groups, _p(out))
    return out


def gemm_i32(X, W):
    """acc[m][n] = sum_k X[m][k] W[n][k] (int8 operands, int32 result)."""
    X = _c(X, np.int8)
    W = _c(W, np.int8)
    M, K = X.shape
    N, K2 = W.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    lib().orc_gemm_i32(_p(X), _p(W), M, N, K, _p(acc))
    return acc


def round_f16(v):
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_round_f16(_p(v), v.size, _p(out))
    return out


def round_bf16(v):
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_round_bf16(_p(v), v.size, _p(out))
    return out


def epilogue_f16(acc, sx, sw):
    """(fp16 bits [M][N] as uint16, unrounded float64 values)."""
    acc = _c(acc, np.int32)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.uint16)
    yd = np.empty((M, N), np.float64)
    lib().orc_epilogue_f16(_p(acc), _p(sx), _p(sw), M, N, _p(y), _p(yd))
    return y, yd


def widen_f16(bits):
    """IEEE binary16 bit patterns -> float32 values (exact: every binary16
    value, subnormals included, is a float32 value)."""
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)


def widen_bf16(bits):
    """bfloat16 bit patterns -> float32 values: bfloat16 is the upper half of
    a float32, so the value is the pattern shifted into the high 16 bits."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_decode(b):
    b = _c(b, np.uint8)
    out = np.empty(b.shape, np.float64)
    lib().orc_e4m3_decode(_p(b), b.size, _p(out))
    return out


def e4m3_encode(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_encode(_p(x), x.size, _p(out))
    return out


def quant_rows_e4m3(x):
    """Per-token FP8 e4m3 activations: (codes u8 [M][K], float32 scales)."""
    x = _c(x, np.float32)
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    s = np.empty(R, np.float32)
    lib().orc_quant_rows_e4m3(_p(x), R, C, _p(q), _p(s))
    return q, s


def int4_sm_codes(q):
    q = _c(q, np.int8)
    out = np.empty(q.shape, np.uint8)
    lib().orc_int4_sm_codes(_p(q), q.size, _p(out))
    return out


def int4_sm_values(codes):
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.int8)
    lib().orc_int4_sm_values(_p(codes), codes.size, _p(out))
    return out


def w4fp8_ref(X8, sx, q, sw):
    """(scaled float64 reference [M][N], exact unscaled sums [M][N])."""
    X8 = _c(X8, np.uint8)
    sx = _c(sx, np.float32)
    q = _c(q, np.int8)
    sw = _c(sw, np.float32)
    M, K = X8.shape
    N = q.shape[0]
    ref = np.empty((M, N), np.float64)
    pre = np.empty((M, N), np.float64)
    lib().orc_w4fp8_ref(_p(X8), _p(sx), _p(q), _p(sw), M, N, K, _p(ref), _p(pre))
    return ref, pre


# ------------------------------------------------------- whole pipelines ----

def w4a8_pack(W, group: int, qmax: int = 127):
    """Offline LiquidQuant of float32 W[N][K]: per-channel INT8, then LQQ."""
    Q, sw = quant_sym_rows(W, qmax)
    codes, s, a, nsat = lqq_encode(Q, group)
    out = {"Q": Q, "sw": sw, "codes": codes, "s_u8": s, "a_u8": a,
           "nsat": nsat, "wq": pack_nibbles(codes)}
    if W.shape[0] % 64 == 0:  # the device format (panel order)
        out["s_panels"] = params_to_panels(s)
        out["a_panels"] = params_to_panels(a)
    return out


def w4fp8_pack(W):
    """INT4 per-channel symmetric weights in sign-magnitude nibbles."""
    q, sw = quant_sym_rows(W, 7)
    codes = int4_sm_codes(q)
    return {"q": q, "sw": sw, "codes": codes, "wq": pack_nibbles(codes)}


def w4fp8g_pack(W, group: int):
    """FP8 variant with per-group scales folded into the FP8 weights
    (oracle section 11): q, s_g [N][K/g], f [N][K/g], t, the folded e4m3
    weights w8 [N][K], sign-magnitude codes and the packed nibbles."""
    W = _c(W, np.float32)
    N, K = W.shape
    G = K // group
    q = np.empty((N, K), np.int8)
    sg = np.empty((N, G), np.float32)
    f = np.empty((N, G), np.float32)
    t = np.empty(1, np.float32)
    lib().orc_w4fp8g_pack(_p(W), N, K, group, _p(q), _p(sg), _p(f), _p(t))
    w8 = np.empty((N, K), np.uint8)
    lib().orc_w4fp8g_weights(_p(q), _p(f), N, K, group, _p(w8))
    codes = int4_sm_codes(q)
    return {"q": q, "sg": sg, "f": f, "t": float(t[0]), "w8": w8, "codes": codes,
            "wq": pack_nibbles(codes)}


def w4fp8g_ref(X8, sx, w8, t: float):
    """(scaled float64 reference [M][N], exact unscaled sums [M][N])."""
    X8 = _c(X8, np.uint8)
    sx = _c(sx, np.float32)
    w8 = _c(w8, np.uint8)
    M, K = X8.shape
    N = w8.shape[0]
    ref = np.empty((M, N), np.float64)
    pre = np.empty((M, N), np.float64)
    lib().orc_w4fp8g_ref(_p(X8), _p(sx), _p(w8), float(t), M, N, K, _p(ref), _p(pre))
    return ref, pre


def w4a8_gemm(X8, sx, pk, group: int):
    """Decoded-weight GEMM: (int32 acc, fp16 bits, unrounded float64)."""
    Qhat = lqq_decode(pk["codes"], pk["s_u8"], pk["a_u8"], group)
    acc = gemm_i32(X8, Qhat)
    y, yd = epilogue_f16(acc, sx, pk["sw"])
    return acc, y, yd


# ----------------------------------------------- W8A8 comparison (section 12)

def pack_w8(Q):
    """INT8 codes [N][K] in the 8-bit tile layout (flat int8 [N*K])."""
    Q = _c(Q, np.int8)
    N, K = Q.shape
    assert N % 16 == 0 and K % 128 == 0
    out = np.empty(N * K, np.int8)
    lib().orc_pack_w8(_p(Q), N, K, _p(out))
    return out


def unpack_w8(packed, N: int, K: int):
    packed = _c(packed, np.int8).reshape(-1)
    assert packed.size == N * K
    Q = np.empty((N, K), np.int8)
    lib().orc_unpack_w8(_p(packed), N, K, _p(Q))
    return Q


def w8a8_pack(W, qmax: int = 127):
    """The first LiquidQuant level alone: per-channel INT8 codes and scales,
    plus their 8-bit tile layout."""
    Q, sw = quant_sym_rows(W, qmax)
    return {"Q": Q, "sw": sw, "wq8": pack_w8(Q)}


def w8a8_gemm(X8, sx, pk):
    """INT8 x INT8 GEMM with the fp16 epilogue: (int32 acc, fp16 bits, float64)."""
    acc = gemm_i32(X8, pk["Q"])
    y, yd = epilogue_f16(acc, sx, pk["sw"])
    return acc, y, yd
