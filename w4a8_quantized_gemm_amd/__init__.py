"""Python binding of libw4a8.so (W4A8 / W4FP8 GEMM for MI355X, gfx950).

Argument marshalling only: every step runs in the HIP kernels of the shared
library.  torch is used for device memory and the current stream.  If the
library is not built, importing this package raises ImportError -- there is
no fallback path.

The C entry points are available unchanged as ``lib.<name>``; the helpers
below take torch tensors, check dtypes/devices/contiguity, and raise
``W4A8Error`` on a non-OK status.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a8.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python w4a8_quantized_gemm_amd/build.py` (hipcc, gfx950)")

# torch carries its own HIP runtime (same soname as the system one).  The
# library must bind to that runtime, since the device pointers and streams it
# receives belong to it: load torch first so the dynamic linker reuses it.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

W4A8_OK = 0
STATUS_NAMES = {0: "W4A8_OK", 1: "W4A8_ERR_NULL_PTR", 2: "W4A8_ERR_SHAPE",
                3: "W4A8_ERR_ALIGNMENT", 4: "W4A8_ERR_WORKSPACE",
                5: "W4A8_ERR_UNSUPPORTED", 6: "W4A8_ERR_HIP"}
PACK_LQQ, PACK_INT4_SYM = 0, 1
OUT_F16, OUT_I32 = 0, 1
OUT_BF16, OUT_F32 = 0, 1
IN_F32, IN_F16, IN_BF16 = 0, 1, 2
ABL_LQQ, ABL_AFFINE16, ABL_LQQ_COARSE = 0, 1, 2
LAYOUT_VERSION = 1

EXPORTS = ("w4a8_pack", "w4a8_quant_act", "w4fp8_quant_act",
           "w4a8_quant_act_ex", "w4fp8_quant_act_ex", "w4a8_workspace_size", "w4a8_gemm",
           "w4a8_gemm_noalloc", "w4a8_gemm_plan",
           "w4a8_gemm_ablation", "w4a8_gemm_grouped", "w4fp8_gemm", "w4fp8g_pack",
           "w4fp8g_gemm", "w8a8_pack", "w8a8_gemm",
           "w4a8_status_str", "w4a8_last_hip_error", "w4a8_layout_version")

_P, _I, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
lib.w4a8_pack.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]
lib.w4a8_quant_act.argtypes = [_P, _I, _I, _P, _P, _P]
lib.w4fp8_quant_act.argtypes = [_P, _I, _I, _P, _P, _P]
lib.w4a8_quant_act_ex.argtypes = [_P, _I, _I, _I, _P, _P, _P]
lib.w4fp8_quant_act_ex.argtypes = [_P, _I, _I, _I, _P, _P, _P]
lib.w4a8_workspace_size.argtypes = [_I, _I, _I, _I]
lib.w4a8_gemm_plan.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P]
lib.w4a8_workspace_size.restype = _Z
lib.w4a8_gemm.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _Z, _P]
lib.w4a8_gemm_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]
lib.w4fp8_gemm.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _Z, _P]
lib.w4a8_gemm_ablation.argtypes = [_I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]
lib.w4a8_gemm_grouped.argtypes = [_P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]
lib.w4fp8g_pack.argtypes = [_P, _I, _I, _I, _P, _P, _P, _P]
lib.w4fp8g_gemm.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _Z, _P]
lib.w8a8_pack.argtypes = [_P, _I, _I, _P, _P, _P]
lib.w8a8_gemm.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _Z, _P]
lib.w4a8_status_str.argtypes = [_I]
lib.w4a8_status_str.restype = ctypes.c_char_p
lib.w4a8_last_hip_error.restype = _I
lib.w4a8_layout_version.restype = _I
for _n in ("w4a8_pack", "w4a8_quant_act", "w4fp8_quant_act", "w4a8_quant_act_ex",
           "w4fp8_quant_act_ex", "w4a8_gemm", "w4a8_gemm_noalloc", "w4a8_gemm_ablation", "w4a8_gemm_grouped",
           "w4fp8_gemm", "w4fp8g_pack", "w4fp8g_gemm", "w8a8_pack", "w8a8_gemm",
           "w4a8_gemm_plan"):
    getattr(lib, _n).restype = _I

assert lib.w4a8_layout_version() == LAYOUT_VERSION


class W4A8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.w4a8_status_str(status).decode()
        extra = ""
        if status == 6:
            extra = f" (hipError {lib.w4a8_last_hip_error()})"
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}{extra}")


def _check(status: int, where: str):
    if status != W4A8_OK:
        raise W4A8Error(status, where)


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _numel_is(t, n, name):
    """Shape checks run before the dtype / device checks, so a caller's
    wrongly sized tensor is named before any pointer reaches the library
    (whose kernels read and write exactly the sizes the shape implies)."""
    if t is not None and t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements, got {t.numel()} "
                         f"(shape {tuple(t.shape)})")


def _shape_is(t, shape, name):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _gemm_shapes(X, sx, packed, out, keys, group=None, E=1):
    """M, N, K of a GEMM call after checking every operand's size against
    them: X [M][K], sx [M], out [M][N], the packed weight arrays of E
    experts (codes, group parameters, channel scales) and K against the
    packed K."""
    if X.dim() != 2:
        raise ValueError("X must be a 2-D tensor [M][K]")
    M, K = X.shape
    N = packed["N"]
    if packed["K"] != K:
        raise ValueError("K of X and of the packed weights differ")
    _numel_is(sx, M, "sx")
    _shape_is(out, (M, N), "out")
    sizes = {"wq": N * K // 2, "wq8": N * K, "sw": N, "tscale": 1}
    if group:
        sizes.update(s_u8=N * K // group, a_u8=N * K // group, fsc=N * K // group)
    for k in keys:
        _numel_is(packed.get(k), E * sizes[k], k)
    return M, N, K


# ------------------------------------------------------------------ API ----

def pack(W, group: int = 64, qmax: int = 127, mode: int = PACK_LQQ, stream=None):
    """w4a8_pack on a float32 [N][K] device tensor.

    Returns a dict with wq (uint8 [N*K/2]), sw (float32 [N]) and, in LQQ
    mode, s_u8 / a_u8 (uint8 [N*K/group], panel order of include/w4a8.h)."""
    torch = _torch()
    _need(W, torch.float32, "W")
    N, K = W.shape
    dev = W.device
    wq = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
    sw = torch.empty(N, dtype=torch.float32, device=dev)
    out = {"wq": wq, "sw": sw, "N": N, "K": K, "mode": mode}
    s_u8 = a_u8 = None
    if mode == PACK_LQQ:
        s_u8 = torch.empty(N * K // group, dtype=torch.uint8, device=dev)
        a_u8 = torch.empty(N * K // group, dtype=torch.uint8, device=dev)
        out.update(s_u8=s_u8, a_u8=a_u8, group=group)
    _check(lib.w4a8_pack(_ptr(W), N, K, group, qmax, mode, _ptr(wq), _ptr(s_u8),
                         _ptr(a_u8), _ptr(sw), _stream(stream)), "w4a8_pack")
    return out


def _in_type(X):
    torch = _torch()
    types = {torch.float32: IN_F32, torch.float16: IN_F16, torch.bfloat16: IN_BF16}
    if X.dtype not in types:
        raise TypeError(f"X: expected float32, float16 or bfloat16, got {X.dtype}")
    _need(X, X.dtype, "X")
    if X.dim() != 2:
        raise ValueError("X must be a 2-D tensor")
    return types[X.dtype]


def _act_outs(X, out, qdtype):
    torch = _torch()
    M, K = X.shape
    if out is None:
        return (torch.empty((M, K), dtype=qdtype, device=X.device),
                torch.empty(M, dtype=torch.float32, device=X.device))
    Xq, sx = out
    _need(Xq, qdtype, "out[0]")
    _need(sx, torch.float32, "out[1]")
    if tuple(Xq.shape) != (M, K) or tuple(sx.shape) != (M,):
        raise ValueError("out tensors must be [M][K] and [M]")
    return Xq, sx


def quant_act(X, stream=None, out=None):
    """Per-token INT8 of float32 / fp16 / bf16 X: (Xq int8 [M][K], sx float32 [M]).

    `out` = (Xq, sx) writes into existing tensors (nothing is allocated, as a
    captured graph needs)."""
    torch = _torch()
    it = _in_type(X)
    M, K = X.shape
    Xq, sx = _act_outs(X, out, torch.int8)
    _check(lib.w4a8_quant_act_ex(_ptr(X), it, M, K, _ptr(Xq), _ptr(sx), _stream(stream)),
           "w4a8_quant_act_ex")
    return Xq, sx


def quant_act_fp8(X, stream=None, out=None):
    """Per-token e4m3 of float32 / fp16 / bf16 X: (Xq uint8 [M][K], sx float32 [M]);
    `out` as for quant_act."""
    torch = _torch()
    it = _in_type(X)
    M, K = X.shape
    Xq, sx = _act_outs(X, out, torch.uint8)
    _check(lib.w4fp8_quant_act_ex(_ptr(X), it, M, K, _ptr(Xq), _ptr(sx), _stream(stream)),
           "w4fp8_quant_act_ex")
    return Xq, sx


def workspace_size(M: int, N: int, K: int, splitk: int = 0) -> int:
    return int(lib.w4a8_workspace_size(M, N, K, splitk))


def gemm_plan(M: int, N: int, K: int, splitk: int = 0) -> dict:
    """The kernel plan w4a8_gemm takes for this shape (host-side, no GPU)."""
    vals = [ctypes.c_int(0) for _ in range(5)]
    _check(lib.w4a8_gemm_plan(M, N, K, splitk, *[ctypes.addressof(v) for v in vals]),
           "w4a8_gemm_plan")
    kernel, rows, chans, splits, parts = (v.value for v in vals)
    return {"kernel": ("stream", "tile16", "tile32")[kernel], "tile_rows": rows,
            "tile_channels": chans, "splits": splits, "k_parts": parts}


def gemm(Xq, sx, packed, out_type: int = OUT_F16, splitk: int = 0, out=None,
         workspace=None, stream=None):
    """w4a8_gemm: Y [M][N] float16 (OUT_F16) or int32 (OUT_I32).

    `workspace` (uint8 device tensor of at least workspace_size() bytes) is
    allocated here when not given and the shape needs one."""
    torch = _torch()
    M, N, K = _gemm_shapes(Xq, sx, packed, out, ("wq", "s_u8", "a_u8", "sw"),
                           packed["group"])
    _need(Xq, torch.int8, "Xq")
    if out_type == OUT_F16 or sx is not None:
        _need(sx, torch.float32, "sx")
    ydt = torch.float16 if out_type == OUT_F16 else torch.int32
    Y = out if out is not None else torch.empty((M, N), dtype=ydt, device=Xq.device)
    _need(Y, ydt, "out")
    if workspace is None:
        need = workspace_size(M, N, K, splitk)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=Xq.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.w4a8_gemm(_ptr(Xq), _ptr(sx), _ptr(packed["wq"]), _ptr(packed["s_u8"]),
                         _ptr(packed["a_u8"]), _ptr(packed["sw"]), _ptr(Y), out_type, M, N,
                         K, packed["group"], splitk, _ptr(workspace), ws_bytes,
                         _stream(stream)), "w4a8_gemm")
    return Y


def gemm_noalloc(Xq, sx, packed, out_type: int = OUT_F16, splitk: int = 0, out=None,
                 stream=None):
    """w4a8_gemm_noalloc: w4a8_gemm with the library's static scratch as the
    split-K workspace (the library allocates nothing; `out` given, nothing
    is allocated here either)."""
    torch = _torch()
    M, N, K = _gemm_shapes(Xq, sx, packed, out, ("wq", "s_u8", "a_u8", "sw"),
                           packed["group"])
    _need(Xq, torch.int8, "Xq")
    if out_type == OUT_F16 or sx is not None:
        _need(sx, torch.float32, "sx")
    ydt = torch.float16 if out_type == OUT_F16 else torch.int32
    Y = out if out is not None else torch.empty((M, N), dtype=ydt, device=Xq.device)
    _need(Y, ydt, "out")
    _check(lib.w4a8_gemm_noalloc(_ptr(Xq), _ptr(sx), _ptr(packed["wq"]), _ptr(packed["s_u8"]),
                                 _ptr(packed["a_u8"]), _ptr(packed["sw"]), _ptr(Y), out_type,
                                 M, N, K, packed["group"], splitk, _stream(stream)),
           "w4a8_gemm_noalloc")
    return Y


def pack_experts(Ws, group: int = 128, stream=None):
    """w4a8_pack of each expert's float32 [N][K] weights, laid end to end as
    w4a8_gemm_grouped expects (Ws: float32 [E][N][K] tensor or list)."""
    torch = _torch()
    parts = [pack(W, group=group, stream=stream) for W in Ws]
    out = {k: torch.cat([p[k] for p in parts]) for k in ("wq", "s_u8", "a_u8", "sw")}
    out.update(N=parts[0]["N"], K=parts[0]["K"], group=group, E=len(parts))
    return out


def gemm_grouped(Xq, sx, offsets, packed, max_rows: int, out_type: int = OUT_F16, out=None,
                 stream=None):
    """w4a8_gemm_grouped: rows offsets[e]..offsets[e+1]-1 of Xq use expert e
    of `packed` (from pack_experts); offsets is a device int32 [E+1] tensor."""
    torch = _torch()
    E = packed["E"]
    M, N, K = _gemm_shapes(Xq, sx, packed, out, ("wq", "s_u8", "a_u8", "sw"),
                           packed["group"], E)
    if offsets.numel() != E + 1:
        raise ValueError("offsets must hold E + 1 entries")
    _need(Xq, torch.int8, "Xq")
    _need(offsets, torch.int32, "offsets")
    if out_type == OUT_F16 or sx is not None:
        _need(sx, torch.float32, "sx")
    ydt = torch.float16 if out_type == OUT_F16 else torch.int32
    Y = out if out is not None else torch.empty((M, N), dtype=ydt, device=Xq.device)
    _need(Y, ydt, "out")
    _check(lib.w4a8_gemm_grouped(_ptr(Xq), _ptr(sx), _ptr(offsets), E, _ptr(packed["wq"]),
                                 _ptr(packed["s_u8"]), _ptr(packed["a_u8"]), _ptr(packed["sw"]),
                                 _ptr(Y), out_type, M, N, K, packed["group"], max_rows,
                                 _stream(stream)), "w4a8_gemm_grouped")
    return Y


def gemm_ablation(variant: int, Xq, sx, packed, out_type: int = OUT_F16, out=None,
                  stream=None):
    """w4a8_gemm_ablation: the matrix-core kernel with decode variant
    ABL_LQQ (production), ABL_AFFINE16 (conventional signed 16-bit-lane
    decode) or ABL_LQQ_COARSE (decode not interleaved with the matrix core)."""
    torch = _torch()
    M, N, K = _gemm_shapes(Xq, sx, packed, out, ("wq", "s_u8", "a_u8", "sw"),
                           packed["group"])
    _need(Xq, torch.int8, "Xq")
    if out_type == OUT_F16 or sx is not None:
        _need(sx, torch.float32, "sx")
    ydt = torch.float16 if out_type == OUT_F16 else torch.int32
    Y = out if out is not None else torch.empty((M, N), dtype=ydt, device=Xq.device)
    _need(Y, ydt, "out")
    _check(lib.w4a8_gemm_ablation(variant, _ptr(Xq), _ptr(sx), _ptr(packed["wq"]),
                                  _ptr(packed["s_u8"]), _ptr(packed["a_u8"]), _ptr(packed["sw"]),
                                  _ptr(Y), out_type, M, N, K, packed["group"], _stream(stream)),
           "w4a8_gemm_ablation")
    return Y


def gemm_fp8(Xq, sx, packed, out_type: int = OUT_BF16, splitk: int = 0, out=None,
             workspace=None, stream=None):
    """w4fp8_gemm: Y [M][N] bfloat16 (OUT_BF16) or float32 (OUT_F32).

    `workspace` as for gemm() (same size: float32 split-K partials)."""
    torch = _torch()
    M, N, K = _gemm_shapes(Xq, sx, packed, out, ("wq", "sw"))
    _need(Xq, torch.uint8, "Xq")
    _need(sx, torch.float32, "sx")
    ydt = torch.bfloat16 if out_type == OUT_BF16 else torch.float32
    Y = out if out is not None else torch.empty((M, N), dtype=ydt, device=Xq.device)
    _need(Y, ydt, "out")
    if workspace is None:
        need = workspace_size(M, N, K, splitk)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=Xq.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.w4fp8_gemm(_ptr(Xq), _ptr(sx), _ptr(packed["wq"]), _ptr(packed["sw"]),
                          _ptr(Y), out_type, M, N, K, splitk, _ptr(workspace), ws_bytes,
                          _stream(stream)), "w4fp8_gemm")
    return Y


def pack_fp8g(W, group: int = 128, stream=None):
    """w4fp8g_pack: INT4 codes with per-group scales folded into FP8.

    Returns a dict with wq (uint8 [N*K/2]), fsc (float32 [K/group][N],
    group-major folded factors) and tscale (float32 [1])."""
    torch = _torch()
    _need(W, torch.float32, "W")
    N, K = W.shape
    dev = W.device
    wq = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
    fsc = torch.empty((K // group, N), dtype=torch.float32, device=dev)
    tscale = torch.empty(1, dtype=torch.float32, device=dev)
    _check(lib.w4fp8g_pack(_ptr(W), N, K, group, _ptr(wq), _ptr(fsc), _ptr(tscale),
                           _stream(stream)), "w4fp8g_pack")
    return {"wq": wq, "fsc": fsc, "tscale": tscale, "N": N, "K": K, "group": group}


def gemm_fp8g(Xq, sx, packed, out_type: int = OUT_BF16, splitk: int = 0, out=None,
              workspace=None, stream=None):
    """w4fp8g_gemm on pack_fp8g output: Y [M][N] bfloat16 or float32."""
    torch = _torch()
    M, N, K = _gemm_shapes(Xq, sx, packed, out, ("wq", "fsc", "tscale"), packed["group"])
    _need(Xq, torch.uint8, "Xq")
    _need(sx, torch.float32, "sx")
    ydt = torch.bfloat16 if out_type == OUT_BF16 else torch.float32
    Y = out if out is not None else torch.empty((M, N), dtype=ydt, device=Xq.device)
    _need(Y, ydt, "out")
    if workspace is None:
        need = workspace_size(M, N, K, splitk)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=Xq.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.w4fp8g_gemm(_ptr(Xq), _ptr(sx), _ptr(packed["wq"]), _ptr(packed["fsc"]),
                           _ptr(packed["tscale"]), _ptr(Y), out_type, M, N, K,
                           packed["group"], splitk, _ptr(workspace), ws_bytes,
                           _stream(stream)), "w4fp8g_gemm")
    return Y


def pack_w8(W, stream=None):
    """w8a8_pack: per-channel INT8 weights in the 8-bit tile layout.

    Returns a dict with wq8 (int8 [N*K]) and sw (float32 [N])."""
    torch = _torch()
    _need(W, torch.float32, "W")
    N, K = W.shape
    wq8 = torch.empty(N * K, dtype=torch.int8, device=W.device)
    sw = torch.empty(N, dtype=torch.float32, device=W.device)
    _check(lib.w8a8_pack(_ptr(W), N, K, _ptr(wq8), _ptr(sw), _stream(stream)), "w8a8_pack")
    return {"wq8": wq8, "sw": sw, "N": N, "K": K}


def gemm_w8a8(Xq, sx, packed, out_type: int = OUT_F16, splitk: int = 0, out=None,
              workspace=None, stream=None):
    """w8a8_gemm on pack_w8 output: Y [M][N] fp16 (OUT_F16) or int32 (OUT_I32)."""
    torch = _torch()
    M, N, K = _gemm_shapes(Xq, sx, packed, out, ("wq8", "sw"))
    _need(Xq, torch.int8, "Xq")
    if out_type == OUT_F16 or sx is not None:
        _need(sx, torch.float32, "sx")
    ydt = torch.float16 if out_type == OUT_F16 else torch.int32
    Y = out if out is not None else torch.empty((M, N), dtype=ydt, device=Xq.device)
    _need(Y, ydt, "out")
    if workspace is None:
        need = workspace_size(M, N, K, splitk)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=Xq.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.w8a8_gemm(_ptr(Xq), _ptr(sx), _ptr(packed["wq8"]), _ptr(packed["sw"]), _ptr(Y),
                         out_type, M, N, K, splitk, _ptr(workspace), ws_bytes, _stream(stream)),
           "w8a8_gemm")
    return Y
