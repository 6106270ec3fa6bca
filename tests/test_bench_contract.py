"""bench.py's host-side contract, checked without a GPU.

- `--gpus N` with N > 1 exits with a message before any device work: the
  routing runs on one GPU here.
- The algorithmic byte counts that the roofline divides by a kernel's time:
  each is the sum of the rows and per-token scalars the kernel must touch once.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_multi_gpu_request_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
    assert p.stdout == ""


def test_block_bytes_per_token():
    T, d, N, S = 16384, 4096, 8, 4
    bf16, f16, f32 = 2, 2, 4
    # Phase 1: read N reps; write h_first (bf16), S-1 state rows (scaled fp16),
    # S*H lse values and one fp32 state scale.
    p1_tok = N * d * bf16 + d * bf16 + (S - 1) * d * f16 + S * 1 * f32 + f32
    # Phase 2: read one state row, H lse values, the scale and the partial; write h_i.
    p2_tok = d * f16 + 1 * f32 + f32 + d * bf16 + d * bf16
    assert (p1_tok, p2_tok) == (98_324, 24_584)
    p1, p2, step = bench.block_bytes(T, d, N, S, 1)
    assert (p1, p2, step) == (T * p1_tok, T * p2_tok, T * (p1_tok + (S - 1) * p2_tok))
    # Eight heads add one lse value per (sublayer, head).
    p1h, p2h, _ = bench.block_bytes(T, d, N, S, 8)
    assert (p1h // T, p2h // T) == (98_436, 24_612)


def test_backward_and_full_bytes_per_token():
    # Block backward: 8 reps, 3 partials and 4 upstream gradients read; 11 gradients written.
    assert bench.bwd_bytes(8192, 4096, 8, 4) == 8192 * (15 + 11) * 4096 * 2
    # Full forward, L = 32: every source read once and every output written once.
    assert bench.full_bytes(4096, 2048, 32) == 4096 * (32 + 32) * 2048 * 2
