"""Host-side checks of the benchmark: the algorithmic byte counts it divides
by are the ones derived from the data layout, and it refuses more than one
GPU.  No GPU is used."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_decode_bytes_per_token_head():
    # state 2 x 64 KiB, inputs (3 d_k + 2 d_v + 1) bf16, window 2 x 3 x 384 bf16,
    # output 128 fp32, per-head parameters (d_k + 4 x 384 + d_v) fp32 over B
    assert bench.decode_bytes_per_token_head(B=64) == 131072 + 1282 + 4608 + 512 + 112
    assert bench.decode_bytes_per_token_head(B=64) == 137586
    # batch 1: the per-head parameters are not amortised
    assert bench.decode_bytes_per_token_head(B=1) == 137474 + 7168


def test_verify_and_commit_bytes():
    assert bench.verify_bytes_per_seq_head(T=8, B=16) == 625360
    # replay records: S0 + window read, inputs, 8 records of 384 x 6 bytes, outputs, parameters
    assert bench.verify_delta_bytes_per_seq_head(T=8, B=16) == 65536 + 2304 + 8 * 1282 + 8 * 2304 + 8 * 512 + 448
    assert bench.commit_delta_bytes_per_seq_head(3) == 131072 + 3 * 1536 + 2 * 2304


def test_prefill_flop_counts_are_positive_and_ordered():
    issued = bench.prefill_mfma_flops_per_chunk_head(128, 128)
    # intra: 240 v_mfma_f32_16x16x32_bf16 (Gram) + 480 v_mfma_f32_16x16x16_bf16
    # ([W | U~]); scan: 1296 of 16x16x32 -- the flops the MFMA instruction
    # counter reads: 476.7 GFLOP per 32768-token call
    x32, x16 = 16 * 16 * 32 * 2, 16 * 16 * 16 * 2
    assert issued == (240 + 1296) * x32 + 480 * x16
    assert issued * (32768 // 64) * 32 == 476741369856
    alg = bench.prefill_algorithmic_flops_per_chunk_head(128, 128)
    assert 0 < alg < issued


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
