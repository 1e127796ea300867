"""The launch path allocates nothing and never synchronises, so a whole window
of decode reads and its flush can be captured in a HIP graph, with the window's
last read either apart or fused into the flush.  Each replay, from the same
starting state, must reproduce the eager run bit for bit; eager work and host
synchronisations sit between the replays."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from workloads import CONFIGS, Workload  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_state_read_amd import binding
    binding.lib()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("fused", [False, True], ids=["apart", "fused"])
@pytest.mark.parametrize("name,B", [("c1", 20), ("c3", 23), ("c4", 19)])
def test_window_replays_match_eager(name, B, fused):
    from rank_state_read_amd.layer import layer_for_workload
    cfg = CONFIGS[name].with_batch(B)
    wl = Workload(cfg)
    lay = layer_for_workload(wl)
    lay.flush(0)
    inputs = [lay.upload_step(wl.step(t)) for t in range(cfg.W)]
    ys = torch.empty((cfg.W, cfg.B, cfg.H, cfg.V), dtype=torch.float32, device="cuda")
    start = (lay.S.clone(), lay.Z.clone())

    def window():
        for pos in range(cfg.W - 1 if fused else cfg.W):
            d = inputs[pos]
            lay.read(pos, d["q"], d["k"], d["v"], d["a"], d["beta"], y=ys[pos])
        if fused:
            d = inputs[cfg.W - 1]
            lay.read_flush(d["q"], d["k"], d["v"], d["a"], d["beta"], y=ys[cfg.W - 1])
        else:
            lay.flush(cfg.W)

    def restore():
        lay.S.copy_(start[0])
        lay.Z.copy_(start[1])
        ys.fill_(float("nan"))

    window()
    torch.cuda.synchronize()
    eager = (ys.clone(), lay.S.clone(), lay.Z.clone())
    assert not torch.isnan(eager[0]).any()

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        window()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref, what in zip((ys, lay.S, lay.Z), eager, ("y", "S", "Z")):
            assert torch.equal(got, ref), f"replay {rep}: {what} differs from the eager run"
        # eager work between replays
        d = inputs[0]
        lay.read(0, d["q"], d["k"], d["v"], d["a"], d["beta"])
        torch.cuda.synchronize()
    how = "fused last read" if fused else "flush"
    print(f"  {name} B={B}: 3 replays of the window's reads + {how} match the eager run", flush=True)
    assert np.isfinite(eager[1].cpu().numpy()).all()
