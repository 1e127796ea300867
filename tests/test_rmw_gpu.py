"""Parity of the standard per-token decode (``sketchssm_rmw_step``) with the
oracle's exact recurrence: every step's y = S_t^T q_t and the state after the
run, for all three layer families, within 1e-4 relative per slab (the same bar
as the sketch path).  The oracle's exact state and y_exact are the ones its pins
check against exact rational arithmetic and the closed forms."""
import sys
import time

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


def _run(wl, steps, items=None, step_source=None, fill_state=None):
    from rank_state_read_amd.layer import layer_for_workload
    c = wl.cfg
    lay = layer_for_workload(wl, with_state=fill_state is None)
    if fill_state is not None:
        fill_state(lay.S)
    src = step_source or wl
    items = items if items is not None else [(b, h) for b in range(c.B) for h in range(c.H)]
    bi = torch.as_tensor([b for b, _ in items])
    hi = torch.as_tensor([h for _, h in items])
    S0 = lay.S[bi, hi].cpu().numpy()
    orc = items_oracle(wl, items, S_init=S0)
    worst = 0.0
    t0 = time.time()
    for t in range(steps):
        st = src.step(t)
        dev = lay.upload_step(st)
        y = lay.rmw_step(dev["q"], dev["k"], dev["v"], dev["a"], dev["beta"])
        so = gather_items(st, items)
        _, ye = orc.read(so["q"], so["k"], so["v"], so["a"], so["beta"])
        if orc.j == c.W:
            orc.flush()  # only the sketch bookkeeping restarts; the exact state runs on
        torch.cuda.synchronize()
        e = _slab_err(y[bi, hi].cpu().numpy(), ye)
        worst = max(worst, e)
        assert e <= TOL, f"y at t={t}: {e:.3e}"
    eS = _slab_err(lay.S[bi, hi].cpu().numpy(), orc.S)
    print(f"  {c.name} B={c.B} steps={steps}: y {worst:.2e}, S {eS:.2e} ({time.time() - t0:.1f}s)",
          flush=True)
    sys.stdout.flush()
    assert eS <= TOL, f"S after {steps} steps: {eS:.3e}"


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,B,steps", [("c0", 2, 40), ("c1", 20, 24), ("c3", 37, 24), ("c4", 37, 24)])
def test_rmw_matches_exact_recurrence(name, B, steps):
    _run(Workload(CONFIGS[name].with_batch(B)), steps)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,kq", [("c1", 8), ("c3", 8), ("c4", 16)])
def test_rmw_shared_key_heads(name, kq):
    import dataclasses
    _run(Workload(dataclasses.replace(CONFIGS[name].with_batch(19), kq_heads=kq)), 20)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c1", "c4"])
def test_rmw_full_size_sampled(name):
    wl = Workload(CONFIGS[name])
    c = wl.cfg
    rng = np.random.default_rng(c.seed + 7)
    items = sorted({(0, 0), (c.B - 1, c.H - 1)} |
                   {(int(rng.integers(c.B)), int(rng.integers(c.H))) for _ in range(30)})
    _run(wl, 6, items=items)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,V,qkv", [("mamba2", 64, "bf16"), ("gdn", 64, "bf16"), ("kda", 80, "bf16"),
                                        ("mamba2", 128, "f32"), ("gdn", 80, "f32"), ("kda", 128, "f32"),
                                        ("mamba2", 112, "bf16"), ("gdn", 96, "bf16"), ("kda", 112, "f32")])
def test_rmw_widths_and_dtypes(kind, V, qkv):
    from workloads import Config
    cfg = Config(f"rmw-{kind}-{V}-{qkv}", kind, B=19, H=8, K=128, V=V, G=2, W=16, steps=20, qkv=qkv,
                 mean_rank=6, rank_cap=49, n_dense=0, seed=79)
    _run(Workload(cfg), 20)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,B", [("c1", 1638), ("c4", 4095)])
def test_rmw_largest_batch(name, B):
    """The largest batch a shape takes (8.6 GB of state), sampled rows across it."""
    from tiled_inputs import TiledRows, tiled_state_fill
    wl = Workload(CONFIGS[name].with_batch(B))
    c = wl.cfg
    small = Workload(CONFIGS[name].with_batch(23))
    rng = np.random.default_rng(c.seed + 11)
    items = sorted({(0, 0), (B - 1, c.H - 1), (B // 2, c.H // 2)} |
                   {(int(rng.integers(B)), int(rng.integers(c.H))) for _ in range(30)})
    _run(wl, 6, items=items, step_source=TiledRows(small, B), fill_state=tiled_state_fill(small, B))
