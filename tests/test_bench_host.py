"""Host-side logic of bench.py, on the CPU: the one-GPU rule, the byte
counts behind the roofline figures, the source digest that decides whether
committed counter summaries still describe the kernels, and the decode
target's outcome."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_weight_and_algorithmic_bytes():
    # 28672 x 8192 at group 128: 4-bit codes plus one UINT8 scale and one
    # UINT8 offset per 128 weights
    assert bench.weight_bytes(28672, 8192, 128) == 28672 * 4096 + 2 * 28672 * 64
    # plus per-channel float32 scales, int8 X, per-token float32 scales and
    # the fp16 output
    M, N, K = 16, 8192, 28672
    assert bench.algo_bytes(M, N, K, 128) == (bench.weight_bytes(N, K, 128) + 4 * N + M * K
                                              + 4 * M + 2 * M * N)


def test_digest_ignores_comments_and_spacing():
    code = 'int f(int a) {\n  return a + 1;  // one more\n}\n/* block\n comment */\n'
    same = 'int f(int a) { return a + 1; }'
    assert bench._code_only(code) == bench._code_only(same)
    # a comment marker inside a string literal is code
    assert "//" in bench._code_only('const char* s = "a//b";')
    # any change to the code changes the text that is hashed
    assert bench._code_only(code) != bench._code_only(code.replace("+ 1", "+ 2"))


def test_source_digest_is_stable():
    assert bench.source_digest() == bench.source_digest()
    assert len(bench.source_digest()) == 64


def test_decode_target_outcome():
    sweep = [{"slot": "upgate:M1", "hbm_frac_algo": 0.71},
             {"slot": "upgate:M16", "hbm_frac_algo": 0.70},
             {"slot": "down:M16", "hbm_frac_algo": 0.69},
             {"slot": "upgate:M128", "hbm_frac_algo": 0.35}]
    v = bench.decode_target(sweep)
    assert v["slots"] == {"upgate:M1": 0.71, "upgate:M16": 0.70, "down:M16": 0.69}
    assert v["met"] is False
    sweep[2]["hbm_frac_algo"] = 0.72
    assert bench.decode_target(sweep)["met"] is True
    assert bench.decode_target([])["met"] is False
