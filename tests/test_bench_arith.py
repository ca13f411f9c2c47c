"""The measurement arithmetic of bench.py, on the host: the byte and flop
counts its rooflines divide by, checked against closed forms written out here
for the Qwen3-8B shape (36 layers, d 4096, 32 q / 8 kv heads of 128, SwiGLU
12288, vocabulary 151936, bf16), and the one-GPU refusal."""
import os
import subprocess
import sys

import numpy as np

import bench
from synth import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SH = workloads.SHAPES["qwen3_8b"]

# per layer: QKV 4096 x (32 + 2 x 8) x 128, O 4096 x 4096, gate and up
# 2 x 12288 x 4096, down 12288 x 4096; LM head 151936 x 4096 (untied)
QKV, O, GU, DOWN, LM = 4096 * 48 * 128, 4096 * 4096, 2 * 12288 * 4096, 12288 * 4096, 151936 * 4096


def test_kv_bytes_per_token():
    # K and V, 8 KV heads of 128 bf16 values, 36 layers
    assert bench.kv_bytes_per_token(SH) == 36 * 2 * 8 * 128 * 2 == 147456


def test_step_roofline_weight_bytes_and_flops():
    """Weight bytes of one draft + verify step: the verify pass reads the
    frozen layers and the LM head once; the draft pass also reads the
    diffusion view's QKV and O matrices (15.136 GB + 18.156 GB)."""
    K, B = 32, 1
    n0 = np.array([512])
    t, byts, flops = bench.step_roofline(SH, B, K, n0)
    frozen = 2 * (36 * (QKV + O + GU + DOWN) + LM)
    verify, draft = frozen, frozen + 2 * 36 * (QKV + O)
    assert verify == 15_136_194_560 and draft == 18_156_093_440
    kv = 2 * (512 + 1 + K) * 147456                 # both passes read [0, n + K] once
    assert byts == verify + draft + kv
    rows = B * (K + 1) + B * K                      # 33 draft rows, 32 verify rows
    assert flops == 2 * rows * (36 * (QKV + O + GU + DOWN) + LM)
    # each class is weight-bound at these row counts: time = bytes / 8 TB/s
    assert abs(t - (verify + draft + kv) / 8e12) < 1e-12


def test_attention_launch_bytes():
    """One layer's attention at 8 x 32768: every visible key's K and V once
    (slots [0, n] and the 32 block keys), plus bf16 queries and outputs."""
    n0 = np.full(8, 32768)
    keys = 8 * (32768 + 1 + 32)
    draft = bench.attn_launch_bytes(SH, 8, 32, n0, "draft")
    assert draft == keys * 8 * 128 * 2 * 2 + 2 * (8 * 33) * 32 * 128 * 2
    verify = bench.attn_launch_bytes(SH, 8, 32, n0, "verify")
    assert verify == keys * 8 * 128 * 2 * 2 + 2 * (8 * 32) * 32 * 128 * 2


def test_prefill_roofline_counts():
    """8 prompts of 32768 tokens in passes of 256 rows per sequence: 128
    passes, causal attention flops 4 x 128 x 32 x 36 x 8 x P (P + 1) / 2."""
    P, B = 32768, 8
    r = bench.prefill_roofline(SH, B, P, 256, 8400.0)
    assert r["passes"] == 128
    assert r["attention_tflop"] == round(4 * 128 * 32 * 36 * B * P * (P + 1) / 2 / 1e12, 1)
    gemm = 2.0 * 36 * (QKV + O + GU + DOWN) * B * P + 2.0 * 4096 * 151936 * B
    assert r["gemm_tflop"] == round(gemm / 1e12, 1)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
