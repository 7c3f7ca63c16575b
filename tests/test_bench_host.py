"""Host-side checks of bench.py: the algorithmic work it prices the kernels
against, its refusal of more than one GPU, and that the committed HBM
counter summary belongs to the committed compressed-branch kernel source.

The local pair count is pinned three ways: a brute-force count over a small
lattice, the closed form per axis (clipped box windows factor over z, y, x),
and the headline figure for a 64^3 lattice with a 3 x 7 x 7 window.
"""

import itertools
import os
import subprocess
import sys

import numpy as np

import bench
import synthgen as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _clipped(n, r):
    """Sum over positions 0..n-1 of the clipped window size along one axis."""
    return sum(min(i + r, n - 1) - max(i - r, 0) + 1 for i in range(n))


def _pairs(w):
    return bench.algorithmic(w)["local_flops"] // (4 * w.n_q_heads * 64)


def test_local_pairs_match_brute_force():
    w = sg.Workload("t", (3, 5, 6), "raster", 4, 2, (3, 5, 5), (1, 1, 2), "f32", "softmax", 1)
    cells = list(itertools.product(range(3), range(5), range(6)))
    want = sum(1 for a in cells for b in cells
               if abs(a[0] - b[0]) <= 1 and abs(a[1] - b[1]) <= 2 and abs(a[2] - b[2]) <= 2)
    assert _pairs(w) == want


def test_headline_counts():
    w = sg.WORKLOADS["block_bf16_64x64x64"]
    assert w.n_tokens == 262144 and w.n_blocks == 16384
    # per-axis closed form: clipped window sizes multiply
    assert _pairs(w) == _clipped(64, 1) * _clipped(64, 3) * _clipped(64, 3) == 36118240
    a = bench.algorithmic(w)
    assert a["global_flops"] == 4 * 262144 * 8 * 16384 * 64          # 8.80 TFLOP
    assert abs(a["global_flops"] / 8.80e12 - 1) < 1e-3
    assert a["global_bwd_flops"] == 10 * 262144 * 8 * 16384 * 64
    # the block pass: K_cmp, V_cmp read; a, cell_to_pos read; K~, V~ and the
    # key norms written; K_loc read, rotated and written (bf16)
    n, hkv, m = 262144, 2, 16384
    assert a["block_pass_bytes"] == (2 * n * hkv * 64 * 2 + n * hkv * 4 + n * 4
                                     + 2 * hkv * m * 64 * 2 + hkv * m * 4 + 2 * n * hkv * 64 * 2)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_committed_counters_belong_to_the_committed_kernel():
    """The HBM traffic bench.py reports comes from profiles/; its source hash
    must match the compressed-branch kernel as committed, or the figure would
    describe another kernel (bench.py then reports null)."""
    t = bench.measured_traffic()
    assert t is not None, "profiles/ holds counters of a different k_global_attn source"
    # at least the algorithmic bytes: Q read, rotated Q and the gated share
    # written (bf16)
    w = sg.WORKLOADS["block_bf16_64x64x64"]
    n, hq = w.n_tokens, w.n_q_heads
    floor = 3 * n * hq * 64 * 2
    assert floor < t < 4 * floor
    assert np.isfinite(t)
