"""The decode's instruction count in the library's own gfx950 code.

LiquidGEMM (Pith review of arXiv 2509.01229, minor comment 1, paper Sec. 5.3)
counts 2 instructions per 4 weights for the dequantisation, 7 per 8 with the
nibble unpack.  On gfx950 one packed dword holds 8 weights; its decode is
  v_and_b32 0x0f0f0f0f, v_lshrrev_b32 4, v_and_b32 0x0f0f0f0f  (unpack: 3)
  v_pk_mad_u16 x 2, v_xor_b32 0x80808080 x 2                   (identity: 4)
The device code of the W4A8 kernels is compiled to assembly here (CPU only)
and the instructions of each kind are counted per kernel: the five counts
must stand in those ratios, and for the 16 x 16 x 64 tile kernel (the large-M
path) their number must be the dwords one loop iteration decodes (two
K-steps x 16 dwords per wave, plus the 8 of the prologue), with one
matrix-core instruction per 16 x 16 x 64 block.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a8_quantized_gemm_amd", "csrc")
OUT = os.path.join(ROOT, "tests", "sanitize", "_build")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")

PATS = {
    "and": r"v_and_b32\S*\s+v\d+,\s*0x0?f0f0f0f,",
    "lshr": r"v_lshrrev_b32\S*\s+v\d+,\s*4,",
    "pkmad": r"v_pk_mad_u16\s",
    "xor": r"v_xor_b32\S*\s+v\d+,\s*0x80808080,",
    "mfma": r"v_mfma_i32_16x16x64_i8\s",
}


def _asm(src):
    out = os.path.join(OUT, os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--offload-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return open(out).read()


def _kernels(asm, marker):
    """{mangled name: counts} for the functions whose name contains marker."""
    out = {}
    for body in re.split(r"\n(?=_Z\S+:)", asm):
        name = body.split(":", 1)[0]
        if name.startswith("_Z") and marker in name:
            out[name] = {k: len(re.findall(p, body)) for k, p in PATS.items()}
    return out


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    srcs = [os.path.join(CSRC, f) for f in ("gemm_mfma16.hip", "gemm_stream.hip")]
    with ThreadPoolExecutor(2) as ex:
        return dict(zip(("tile16", "stream"), ex.map(_asm, srcs)))


def _ratios_hold(c):
    # per decoded dword: 2 and, 1 shift, 2 multiply-adds, 2 XOR (a stray
    # shift by 4 elsewhere in a kernel is allowed)
    d = c["pkmad"] // 2
    return (c["pkmad"] == 2 * d and c["xor"] == 2 * d and c["and"] == 2 * d
            and d <= c["lshr"] <= d + 1)


def test_tile16_decode_is_seven_per_eight(asm):
    ks = {n: c for n, c in _kernels(asm["tile16"], "w4a8_mfma16_kernel").items()
          if re.search(r"Lb0ELi[12]EEEv", n)}  # LiquidQuant kinds (W8 = false), K parts 1 or 2
    assert len(ks) >= 14
    for name, c in ks.items():
        mt = 256 if "ILi256E" in name else 128
        assert _ratios_hold(c), (name, c)
        # one loop iteration runs two K-steps of 16 dwords per wave, the
        # prologue decodes 8 more
        assert c["pkmad"] == 2 * (2 * 16 + 8), (name, c)
        # two K-steps of MT/16 row blocks x 4 channel blocks x 2 halves
        assert c["mfma"] == 2 * (mt // 16) * 4 * 2, (name, c)


def test_stream_decode_is_seven_per_eight(asm):
    ks = {n: c for n, c in _kernels(asm["stream"], "w4a8_stream_kernel").items()
          if c["pkmad"] > 0}
    assert len(ks) >= 16
    for name, c in ks.items():
        assert _ratios_hold(c), (name, c)
