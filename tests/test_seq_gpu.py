"""Continuous batching through the C ABI: every sequence has its own window
phase.  Sequences join at different steps (their first sketch formed by a
0-token flush of their row), read at their own window position, are flushed
alone when their window fills, one is flushed early with a partial window, and
some sit idle (position -1) for a while.  Every active output, and each
flushed row's state and sketch, is compared with the oracle driven one
sequence at a time (each sequence's window counter is its own), within 1e-4
relative per slab; idle rows must leave y untouched."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import gather_items, items_oracle  # noqa: E402
from workloads import CONFIGS, Workload  # noqa: E402

TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_state_read_amd import binding
    binding.lib()


def _slab_err(got, ref):
    got = np.asarray(got, np.float64).reshape(len(ref), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((np.abs(got - ref).max(axis=1) / den).max())


def _schedule(B, T, W, seed):
    """join step, idle span and one early flush per sequence (deterministic)."""
    rng = np.random.default_rng(seed)
    join = rng.integers(0, W // 2, size=B)
    join[0] = 0
    idle = {}
    for b in rng.choice(B, size=max(1, B // 4), replace=False):
        s0 = int(rng.integers(W // 2, T - 4))
        idle[int(b)] = (s0, s0 + int(rng.integers(1, 5)))
    early = {int(b): int(rng.integers(W // 2, T - 2)) for b in rng.choice(B, size=max(1, B // 5), replace=False)}
    return join, idle, early


def _run(name, B, T, kq=None, V=None):
    import dataclasses
    from rank_state_read_amd.layer import layer_for_workload
    cfg = dataclasses.replace(CONFIGS[name].with_batch(B), kq_heads=kq)
    if V is not None:
        cfg = dataclasses.replace(cfg, V=V)
    wl = Workload(cfg)
    W, H = cfg.W, cfg.H
    lay = layer_for_workload(wl)
    S_init = lay.S.cpu().numpy()
    orcs = [items_oracle(wl, [(b, h) for h in range(H)], S_init=S_init[b]) for b in range(B)]
    join, idle, early = _schedule(B, T, W, cfg.seed)
    pos = np.full(B, -1, np.int64)
    dev = torch.device("cuda")
    worst = {"y": 0.0, "S": 0.0, "Z": 0.0}

    def check_rows(rows):
        if not rows:
            return
        S = lay.S.cpu().numpy()
        for b in rows:
            e = _slab_err(S[b], orcs[b].S0)
            worst["S"] = max(worst["S"], e)
            assert e <= TOL, f"S of row {b}: {e:.3e}"
            for h in range(H):
                r = int(wl.ranks[h])
                if r == 0:
                    continue
                e = _slab_err(lay.z_item(b, h).cpu().numpy()[None], orcs[b].Z[h, :r][None])
                worst["Z"] = max(worst["Z"], e)
                assert e <= TOL, f"Z of row {b} head {h}: {e:.3e}"

    def flush(rows, counts):
        seqs = torch.tensor(rows, dtype=torch.int32, device=dev)
        ntok = torch.tensor(counts, dtype=torch.int32, device=dev)
        lay.flush_seq(seqs, ntok)
        torch.cuda.synchronize()

    for t in range(T):
        joining = [b for b in range(B) if join[b] == t]
        if joining:                      # first sketch of each joining sequence, S untouched
            flush(joining, [0] * len(joining))
            for b in joining:
                pos[b] = 0
            check_rows(joining)
        active = [b for b in range(B) if pos[b] >= 0 and not (b in idle and idle[b][0] <= t < idle[b][1])]
        p_dev = np.full(B, -1, np.int32)
        for b in active:
            p_dev[b] = pos[b]
        st = wl.step(t)
        d = lay.upload_step(st)
        lay.y.fill_(float("nan"))
        y = lay.read_seq(torch.from_numpy(p_dev).to(dev), d["q"], d["k"], d["v"], d["a"], d["beta"])
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        for b in range(B):
            if b in active:
                so = gather_items(st, [(b, h) for h in range(H)])
                yo, _ = orcs[b].read(so["q"], so["k"], so["v"], so["a"], so["beta"])
                e = _slab_err(yh[b], yo)
                worst["y"] = max(worst["y"], e)
                assert e <= TOL, f"y of row {b} at t={t} (pos {pos[b]}): {e:.3e}"
            else:
                assert np.isnan(yh[b]).all(), f"idle row {b} was written at t={t}"
        full, part = [], []
        for b in active:
            pos[b] += 1
            if pos[b] == W:
                full.append(b)
            elif early.get(b) == t:
                part.append(b)
        if full or part:
            flush(full + part, [W] * len(full) + [int(pos[b]) for b in part])
            for b in full + part:
                orcs[b].flush()
                pos[b] = 0
            check_rows(full + part)
    print(f"  {name} B={B} T={T}: max errors {worst}", flush=True)
    sys.stdout.flush()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,B,kq", [("c1", 20, None), ("c1", 37, 8), ("c3", 19, None), ("c4", 19, 16),
                                       ("c0", 2, None)])
def test_staggered_windows(name, B, kq):
    _run(name, B, 2 * CONFIGS[name].W + 9, kq)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,V", [("c1", 96), ("c3", 112), ("c4", 96)])
def test_staggered_windows_other_value_widths(name, V):
    """Value widths between the headline layers' (every multiple of 16 from 64 to 128 is accepted)."""
    _run(name, 19, 2 * CONFIGS[name].W + 9, V=V)
