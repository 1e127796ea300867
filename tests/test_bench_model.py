"""The benchmark's host side: its algorithmic byte model and its refusal of
more than one GPU.  The per-step totals below were derived by hand from the
layer shapes (state K x V fp32, sketch r x V fp32, bf16 q/k/v, fp32 decay,
beta and y; 7.5 buffered tokens read plus one appended per read on average)
and are independent of bench.py's code; bench.py adds the coefficient maps,
read once per launch, on top of them."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import CONFIGS, Workload  # noqa: E402

# MB per read launch, averaged over the 16 window positions: sketch path
# (without the coefficient maps) and full-state-read baseline
HAND_TOTALS = {"c1": (222.5, 1491.8), "c2": (1248.0, 2983.6), "c3": (71.9, 583.6), "c4": (318.3, 1246.3)}


def _frame_bytes(cfg, ranks):
    per_group = cfg.H // cfg.G
    frames = {(h // per_group, int(ranks[h])) for h in range(cfg.H) if ranks[h] > 0}
    return sum(r for _, r in frames) * cfg.K * 4


@pytest.mark.parametrize("name", sorted(HAND_TOTALS))
def test_read_bytes_match_hand_totals(name):
    cfg = CONFIGS[name]
    ranks = Workload(cfg).ranks
    sketch = np.mean([bench.read_bytes(cfg, ranks, p) for p in range(cfg.W)])
    dense = np.mean([bench.read_bytes(cfg, ranks, p, dense_all=True) for p in range(cfg.W)])
    want_sketch, want_dense = HAND_TOTALS[name]
    assert abs((sketch - _frame_bytes(cfg, ranks)) / 1e6 - want_sketch) < 0.1
    assert abs(dense / 1e6 - want_dense) < 0.1


def test_flush_bytes_at_the_nano_layer():
    """c1: state read and written (2 x 1.342 GB), the 16-token window (420 B
    per token and item), the sketch written (6 rows of 320 B per sketch item
    on average) and the basis rows (once per head)."""
    cfg = CONFIGS["c1"]
    ranks = Workload(cfg).ranks
    items = cfg.B * cfg.H
    want = (items * (2 * 128 * 80 * 4 + 16 * 420) + cfg.B * 320 * int(ranks.sum())
            + 128 * 4 * int(ranks.sum()))
    assert bench.flush_bytes(cfg, ranks, cfg.W) == want
    assert abs(bench.flush_bytes(cfg, ranks, cfg.W) / 1e9 - 2.97) < 0.01
    # a 0-token flush (the initial sketch) reads the sketch heads' states only
    n_sketch = int((ranks > 0).sum())
    assert bench.flush_bytes(cfg, ranks, 0) == (cfg.B * n_sketch * 128 * 80 * 4 + cfg.B * 320 * int(ranks.sum())
                                                + 128 * 4 * int(ranks.sum()))


def test_standard_decode_bytes_at_the_nano_layer():
    """Read and write of the 40 KB state, q, k, v, decay in and y out per item."""
    cfg = CONFIGS["c1"]
    assert bench.rmw_bytes(cfg) == cfg.B * cfg.H * (2 * 40960 + 256 + 256 + 160 + 4 + 320)


def test_read_launch_write_bytes():
    """What a read launch writes: y (V fp32) and the appended token (k, v bf16,
    decay and beta fp32) of every item; c1 24.2 MB, c3 (Gated DeltaNet, K = V =
    128) 256 x 32 x (512 + 256 + 256 + 4 + 4) B."""
    c1, c3 = CONFIGS["c1"], CONFIGS["c3"]
    assert bench.read_write_bytes(c1) == 256 * 128 * (320 + 256 + 160 + 4)
    assert bench.read_write_bytes(c3) == 256 * 32 * (512 + 256 + 256 + 4 + 4)


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
def test_matched_probe_launches_fit_the_probe(name):
    """The probe launches that stand for each window position's read: whole
    64 KB chunks, a mix the probe accepts, and never more than one 1 GiB probe
    source (c2's reads pass 1 GiB at high positions)."""
    cfg = CONFIGS[name]
    ranks = Workload(cfg).ranks
    w = bench.read_write_bytes(cfg)
    for p in range(cfg.W):
        rd, m = bench.matched_probe(bench.read_bytes(cfg, ranks, p), w)
        assert m in (2, 4, 8, 16)
        assert 0 < rd <= bench.STREAM_BYTES and rd % (16 * 4096) == 0
        assert rd % m == 0 and (rd // m) % 4096 == 0
    # c1 at window position 0 reads 95 MB and writes 24 MB: about 4 reads per write
    rd, m = bench.matched_probe(bench.read_bytes(CONFIGS["c1"], Workload(CONFIGS["c1"]).ranks, 0),
                                bench.read_write_bytes(CONFIGS["c1"]))
    assert m == 4 and abs(rd / 1e6 - 95.4) < 0.5


@pytest.mark.timeout(300)
def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=280)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
