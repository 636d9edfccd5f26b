"""Host logic of bench.py, without a GPU: the single-GPU contract, the
algorithmic units the roofline divides by (closed forms of the layer's work
and of the bytes each kernel must move), and the rocprofv3 commands it
generates (counter passes within what one pass can collect, the program
after `--`, only committed files run)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


def test_linear_flops_closed_form():
    # 4 M N K (forward, dX) + 6 M r (N + K) (T, U, the adapter terms, dA, dB)
    M, N, K, r = 2048, 4096, 4096, 16
    assert bench.linear_flops(M, N, K, r) == 4 * M * N * K + 6 * M * r * (N + K)
    assert bench.linear_flops(M, N, K, r) == 139_049_566_208
    # the 11008-wide MLP block: three linears of 4096 tokens, r = 64
    mlp = 2 * bench.linear_flops(4096, 11008, 4096, 64) + bench.linear_flops(4096, 4096, 11008, 64)
    assert round(mlp / 1e9, 1) == 2287.5


def test_weight_and_gemv_bytes():
    # NF4 storage: N K / 2 packed bytes, one 8-bit code per 64-block, one fp32
    # scale per 256 codes, one fp32 mean
    N, K = 28672, 8192
    assert bench.weight_bytes(N, K) == N * K // 2 + N * K // 64 + 4 * (N * K // 64 // 256) + 4
    # the small-M forward kernel adds X, B, T and Y: 122.16 / 122.38 / 123.27 MB
    got = [bench.gemv_bytes(M, N, K, 16) for M in (1, 4, 16)]
    assert [round(b / 1e6, 2) for b in got] == [122.16, 122.38, 123.27]
    assert bench.algorithmic_bytes("gemv", 1) == got[0]


def test_gemm_operand_bytes():
    M, N, K, r = 2048, 4096, 4096, 16
    w = bench.weight_bytes(N, K)
    assert bench.algorithmic_bytes("fwd_gemm") == 2 * M * K + w + 2 * M * r + 2 * N * r + 2 * M * N
    assert bench.algorithmic_bytes("dx_gemm") == 2 * M * N + 2 * N * K + 2 * M * r + 2 * r * K + 2 * M * K
    assert bench.algorithmic_bytes("dequant") == w + 2 * N * K


# rocprofv3 collects one pass per run; these are the per-block limits of a pass.
LIMITS = {"SQ_": 8, "TA_": 2, "TD_": 2, "GRBM_": 2, "TCP_": 4}


def test_profile_commands_fit_one_pass_each():
    cmds = bench.profile_commands("/tmp/prof_out")
    assert {"kt", "f", "w"} <= set(cmds)
    me = os.path.abspath(os.path.join(ROOT, "bench.py"))
    for name, cmd in cmds.items():
        words = cmd.split()
        assert words[0] == "rocprofv3", name
        prog = words[words.index("--") + 1:]
        assert prog[0] == "python3" and os.path.abspath(prog[1]) == me, name   # program after --
        assert "_work" not in cmd
        if "--pmc" not in words:
            continue
        ctrs = words[words.index("--pmc") + 1:words.index("--output-format")]
        for prefix, most in LIMITS.items():
            assert sum(c.startswith(prefix) for c in ctrs) <= most, (name, prefix)
        if "FETCH_SIZE" in ctrs or "WRITE_SIZE" in ctrs:
            assert len(ctrs) == 1, name   # the TCC-derived sizes each get a run of their own
        assert "--sys-trace" not in words and "--runtime-trace" not in words


@pytest.mark.parametrize("flag", ["--profile-commands"])
def test_profile_commands_cli_prints_one_command_per_line(flag, tmp_path):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), flag, str(tmp_path)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == len(bench.profile_commands(str(tmp_path)))
    assert all(l.startswith("rocprofv3 ") for l in lines)
