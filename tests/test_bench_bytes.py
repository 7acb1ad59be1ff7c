"""The compulsory byte counts behind every roofline fraction bench.py prints,
checked against the tensor sizes of each workload written out here, plus
the benchmark's refusal of more than one GPU and its rule for measured
traffic (reported only for the kernel source it was measured on).  CPU
only."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BF16, F32 = 2, 4


def test_prefill_bytes():
    B, T, H, d = 4, 2048, 16, 128
    tok = B * T * H
    qkvo = 4 * tok * d * BF16              # q, k, v read, o written
    alpha = tok * d * F32                  # one fp32 gate per key channel
    beta = tok * F32
    s_final = B * H * d * d * F32          # S0 absent
    assert qkvo + alpha + beta + s_final == 206_045_184
    assert bench.prefill_bytes(B, T, H, d, d) == 206_045_184


def test_long_context_bytes():
    B, T, H, d = 1, 65536, 32, 128
    tok = B * T * H
    total = 4 * tok * d * BF16 + tok * d * F32 + tok * F32 + 2 * B * H * d * d * F32   # S0 read too
    assert total == 3_233_808_384
    assert bench.prefill_bytes(B, T, H, d, d, s0=True) == total


def test_packed_bytes():
    # the seeded draw of the packed-batch workload: 274,797 tokens, 64 sequences
    T, N, H, d = 274_797, 64, 16, 128
    per_tok = 4 * d * BF16 + d * F32 + F32
    total = T * H * per_tok + 2 * N * H * d * d * F32
    assert total == 6_905_215_808
    assert bench.packed_bytes(T, N, H, d, d) == total


def test_gate_form_bytes():
    B, T, H, d = 4, 2048, 16, 128
    tok = B * T * H
    base = 4 * tok * d * BF16 + tok * F32 + B * H * d * d * F32
    assert bench.prefill_bytes(B, T, H, d, d, gate_form="scalar") == base + tok * F32
    assert bench.prefill_bytes(B, T, H, d, d, gate_form="none") == base
    assert bench.prefill_bytes(B, T, H, d, d, gate_form="log_channel") == base + tok * d * F32


def test_decode_bytes():
    N, H, d = 256, 32, 128
    per_unit = 2 * d * d * F32 + 4 * d * BF16 + d * F32 + F32   # state in and out; q, k, v, o; alpha; beta
    assert per_unit == 132_612
    assert N * H * per_unit == 1_086_357_504
    assert bench.decode_bytes(N, H, d, d) == 1_086_357_504


def test_decode_tokens_bytes():
    N, H, d, Tk = 256, 32, 128, 4
    per_unit = 2 * d * d * F32 + Tk * (4 * d * BF16 + d * F32 + F32)
    assert per_unit == 137_232
    assert bench.decode_tokens_bytes(N, H, d, d, Tk) == N * H * per_unit == 1_124_204_544


def test_prefill_flops():
    # 6 d_k d_v + 2C(3 d_k + 2 d_v) + C^2/3 per head-token at C = 64, d = 128
    per = 6 * 128 * 128 + 2 * 64 * (3 * 128 + 2 * 128) + 64 * 64 / 3
    assert round(per) == 181_589
    assert bench.prefill_flops(4, 2048, 16, 128, 128) == 4 * 2048 * 16 * per


def test_measured_traffic_needs_the_measured_source(monkeypatch):
    key = "prefill"
    fname, sha, nbytes = bench.MEASURED_TRAFFIC[key]
    assert os.path.exists(os.path.join(ROOT, "linear_attention_kda_amd", "csrc", fname))
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, key, (fname, "0" * 16, nbytes))
    assert bench.measured_traffic(key) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
