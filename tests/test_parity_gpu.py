"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every decode step's y, and S and Z after every flush, are compared with the
float64 oracle on the same seeded inputs.  The bar is a relative error of 1e-4
per slab, max |gpu - ref| / max |ref|, where a slab is one (t, b, h) output
vector, one item's K x V state or one item's r x V sketch; integer tables are
compared bit for bit in the CPU tests.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import gather_items, items_oracle  # noqa: E402
from workloads import CONFIGS, Config, Workload  # noqa: E402
from tiled_inputs import TiledRows, tiled_state_fill  # noqa: E402
from parity_run import TOL, Run, _log, _run_steps, _sample_items, _slab_err  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_state_read_amd import binding
    binding.lib()


# ---------------------------------------------------------------------------
# every output of reduced batches (two full tiles of 16 rows and a ragged tail)
# ---------------------------------------------------------------------------
@pytest.mark.timeout(300)
def test_c0_all_steps():
    _run_steps(Workload(CONFIGS["c0"]), CONFIGS["c0"].steps)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,B,steps", [("c1", 20, 48), ("c2", 20, 40), ("c3", 37, 48),
                                          ("c4", 37, 48)])
def test_reduced_batch_all_items(name, B, steps):
    _run_steps(Workload(CONFIGS[name].with_batch(B)), steps)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,kq,B,steps", [("c1", 8, 20, 40), ("c3", 8, 19, 36), ("c4", 16, 19, 36),
                                             ("c0", 2, 2, 40)])
def test_shared_key_heads(name, kq, B, steps):
    """q, k and the window's keys shared by H / kq consecutive heads."""
    import dataclasses
    cfg = dataclasses.replace(CONFIGS[name].with_batch(B), kq_heads=kq)
    _run_steps(Workload(cfg), steps)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,kq", [("c1", 8), ("c4", 16)])
def test_shared_key_heads_dense_baseline(name, kq):
    import dataclasses
    cfg = dataclasses.replace(CONFIGS[name].with_batch(19), kq_heads=kq)
    wl = Workload(cfg)
    wl0 = Workload(cfg, ranks=np.zeros(cfg.H, np.int32), basis=wl.basis)
    _run_steps(wl0, cfg.W + 5, dense_baseline=True, step_source=wl)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["c1", "c3", "c4"])
def test_long_run_drift(name):
    """Many windows on a few items: errors must not grow with the flush count."""
    cfg = CONFIGS[name].with_batch(3)
    wl = Workload(cfg)
    hs = [int(np.argmax(wl.ranks)), int(np.argmin(wl.ranks)), 0]
    items = [(b, h) for b in range(3) for h in hs]
    _run_steps(wl, 12 * cfg.W, items=items)


# ---------------------------------------------------------------------------
# full sizes, in the launch configuration the benchmark times, sampled items
# ---------------------------------------------------------------------------
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_full_size_sampled(name):
    cfg = CONFIGS[name].with_steps(CONFIGS[name].W + 4)
    wl = Workload(cfg)
    items = _sample_items(wl)
    _log(f"  {name}: full size B={cfg.B}, {len(items)} sampled items")
    _run_steps(wl, cfg.steps, items=items)


# ---------------------------------------------------------------------------
# the dense-read baseline
# ---------------------------------------------------------------------------
@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,B", [("c1", 20), ("c3", 19), ("c4", 19), ("c0", 2)])
def test_dense_read_baseline(name, B):
    cfg = CONFIGS[name].with_batch(B)
    wl = Workload(cfg)
    wl0 = Workload(cfg, ranks=np.zeros(cfg.H, np.int32), basis=wl.basis)
    _run_steps(wl0, 2 * cfg.W + 3, dense_baseline=True, step_source=wl)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,B", [("c1", 20), ("c4", 19)])
@pytest.mark.parametrize("kind", ["head", "low-first"])
def test_other_launch_orders(name, B, kind):
    """A plan made with sketchssm_plan_create_ordered: the oracle's outputs, and
    bit for bit those of the planner's own order (no item depends on the order)."""
    import torch
    from rank_state_read_amd.layer import launch_order
    wl = Workload(CONFIGS[name].with_batch(B))
    steps = wl.cfg.W + 3
    ref = _run_steps(wl, steps, fused=True)
    got = _run_steps(wl, steps, fused=True, order=launch_order(wl.ranks, kind))
    assert torch.equal(got.lay.S, ref.lay.S) and torch.equal(got.lay.Z, ref.lay.Z)
    assert torch.equal(got.lay.y, ref.lay.y)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def _edge_cfg(kind, V, B=19, cap=49, qkv="bf16"):
    return Config(f"edge-{kind}-{V}", kind, B=B, H=8, K=128, V=V, G=2, W=16, steps=40,
                  qkv=qkv, mean_rank=6, rank_cap=cap, n_dense=0, seed=77)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,V", [("mamba2", 80), ("mamba2", 64), ("mamba2", 128), ("gdn", 128),
                                    ("gdn", 80), ("gdn", 64), ("kda", 128), ("kda", 80), ("kda", 64),
                                    ("mamba2", 96), ("mamba2", 112), ("gdn", 96), ("gdn", 112),
                                    ("kda", 96), ("kda", 112)])
def test_rank_extremes(kind, V):
    """Ranks at 1, at tile edges (16, 17, 32, 33), at the cap, mixed with dense heads."""
    cfg = _edge_cfg(kind, V, cap=64)
    ranks = np.array([1, 16, 0, 17, 64, 33, 49, 0], np.int32)
    _run_steps(Workload(cfg, ranks=ranks), 2 * cfg.W + 5)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,V", [("mamba2", 80), ("gdn", 128), ("kda", 128)])
def test_small_odd_largest_rank(kind, V):
    """A plan whose largest rank is odd and below 16 (the coefficient map's LDS
    piece then has an odd row count)."""
    cfg = _edge_cfg(kind, V)
    ranks = np.array([1, 3, 5, 0, 5, 3, 1, 2], np.int32)
    _run_steps(Workload(cfg, ranks=ranks), cfg.W + 5)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,V", [("mamba2", 80), ("gdn", 128), ("kda", 128)])
def test_single_sequence_all_dense_and_all_sketch(kind, V):
    cfg = _edge_cfg(kind, V, B=1)
    _run_steps(Workload(cfg, ranks=np.zeros(8, np.int32)), cfg.W + 3)
    _run_steps(Workload(cfg, ranks=np.array([3, 5, 7, 9, 11, 13, 15, 49], np.int32)), cfg.W + 3)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,V", [("mamba2", 80), ("gdn", 128), ("kda", 128)])
def test_flush_without_tokens_keeps_state_bitwise(kind, V):
    cfg = _edge_cfg(kind, V)
    wl = Workload(cfg)
    r = Run(wl)
    before = r.lay.S.clone()
    r.init_sketch()                     # flush(n_tokens = 0): Z only
    assert torch.equal(before, r.lay.S)
    for _ in range(5):
        r.step()
    before = r.lay.S.clone()
    r.lay.flush(0)
    torch.cuda.synchronize()
    assert torch.equal(before, r.lay.S)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,V", [("mamba2", 80), ("gdn", 128), ("kda", 128)])
def test_partial_window_flush(kind, V):
    """Flush after 5 tokens, then keep decoding from window slot 0."""
    cfg = _edge_cfg(kind, V)
    wl = Workload(cfg)
    r = Run(wl)
    r.init_sketch()
    for _ in range(5):
        r.step()
    r.lay.flush(5)
    r.orc.flush()
    torch.cuda.synchronize()
    r.check_S()
    r.check_Z()
    # continue: the next window starts at slot 0
    base = r.t
    for _ in range(cfg.W + 2):
        c = cfg
        st = wl.step(r.t)
        dev = r.lay.upload_step(st)
        pos = (r.t - base) % c.W
        y = r.lay.read(pos, dev["q"], dev["k"], dev["v"], dev["a"], dev["beta"])
        if pos == c.W - 1:
            r.lay.flush(c.W)
        so = gather_items(st, r.items)
        yo, _ = r.orc.read(so["q"], so["k"], so["v"], so["a"], so["beta"])
        torch.cuda.synchronize()
        yg = y[torch.as_tensor(r.bi), torch.as_tensor(r.hi)].cpu().numpy()
        assert _slab_err(yg, yo) <= TOL
        r.t += 1
        if r.orc.j == c.W:
            r.orc.flush()
            r.check_S()
            r.check_Z()


@pytest.mark.timeout(300)
def test_bitwise_reproducible():
    cfg = CONFIGS["c4"].with_batch(5)
    outs = []
    for _ in range(2):
        from rank_state_read_amd.layer import layer_for_workload
        wl = Workload(cfg)
        lay = layer_for_workload(wl)
        lay.flush(0)
        ys = []
        for t in range(cfg.W + 2):
            dev = lay.upload_step(wl.step(t))
            ys.append(lay.read(t % cfg.W, dev["q"], dev["k"], dev["v"], dev["a"], dev["beta"]).clone())
            if t % cfg.W == cfg.W - 1:
                lay.flush(cfg.W)
        torch.cuda.synchronize()
        outs.append((torch.stack(ys), lay.S.clone(), lay.Z.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


@pytest.mark.timeout(120)
def test_sketch_heads_do_not_read_the_state():
    """Sketch heads' outputs do not depend on S between flushes (only dense heads read it)."""
    from rank_state_read_amd.layer import layer_for_workload
    cfg = CONFIGS["c1"].with_batch(4)
    wl = Workload(cfg)
    lay = layer_for_workload(wl)
    lay.flush(0)
    dev = lay.upload_step(wl.step(0))
    y1 = lay.read(0, dev["q"], dev["k"], dev["v"], dev["a"], dev["beta"]).clone()
    lay.S.fill_(float("nan"))
    y2 = lay.read(0, dev["q"], dev["k"], dev["v"], dev["a"], dev["beta"]).clone()
    torch.cuda.synchronize()
    sk = torch.as_tensor(wl.ranks > 0)
    assert torch.equal(y1[:, sk], y2[:, sk])
    assert torch.isnan(y2[:, ~sk]).all()


class _SpecialTokens:
    """Wraps a workload's step stream and replaces chosen tokens with the
    degenerate values of the recurrence: a full reset (decay 0), no decay
    (decay 1), no write (beta 0, or a zero key for Mamba-2), a zero key, a zero
    value and a zero query (whose output must be exactly 0).  A reset at the
    last slot of a window leaves a rank-1 state at the flush, whose sketch rows
    can cancel; the Z check then uses the fp32 error bound (see Run)."""

    EDITS = {2: "a0", 4: "a1", 6: "nowrite", 8: "k0", 10: "v0", 12: "q0", 15: "a0", 20: "a0",
             31: "nowrite"}

    def __init__(self, wl):
        self.wl = wl

    def step(self, t):
        st = dict(self.wl.step(t))
        edit = self.EDITS.get(t)

        def zero(key):
            st[key] = np.zeros_like(st[key])
            if st.get(key + "_bits") is not None:
                st[key + "_bits"] = np.zeros_like(st[key + "_bits"])

        if edit == "a0":
            st["a"] = np.zeros_like(st["a"])
        elif edit == "a1":
            st["a"] = np.ones_like(st["a"])
        elif edit == "nowrite":
            if st.get("beta") is not None:
                st["beta"] = np.zeros_like(st["beta"])
            else:
                zero("k")
        elif edit in ("k0", "v0", "q0"):
            zero(edit[0])
        return st


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,V", [("mamba2", 80), ("gdn", 128), ("kda", 128)])
def test_degenerate_tokens(kind, V):
    cfg = _edge_cfg(kind, V)
    wl = Workload(cfg, ranks=np.array([0, 3, 6, 16, 17, 0, 49, 1], np.int32))
    r = Run(wl, step_source=_SpecialTokens(wl), z_error_bound=True)
    r.init_sketch()
    for t in range(2 * cfg.W + 3):
        r.step()
    _log(f"  {kind}: degenerate tokens, max errors {r.max_err}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,V", [("mamba2", 80), ("gdn", 128), ("kda", 64)])
@pytest.mark.parametrize("B", [16, 17])
def test_single_head(kind, V, B):
    """A layer of one head: exactly one 16-row tile, or one and a ragged row;
    as a sketch head and as a dense head, with the window's last read apart
    from its flush and fused into it."""
    cfg = Config(f"edge-h1-{kind}", kind, B=B, H=1, K=128, V=V, G=1, W=16, steps=20, qkv="bf16",
                 mean_rank=7, rank_cap=49, n_dense=0, seed=79)
    for r in (7, 0):
        for fused in (False, True):
            _run_steps(Workload(cfg, ranks=np.array([r], np.int32)), cfg.W + 2, fused=fused)


@pytest.mark.timeout(300)
def test_max_heads():
    """256 heads (the largest the head table indexes), dense heads among them."""
    cfg = Config("edge-h256", "mamba2", B=3, H=256, K=128, V=64, G=16, W=16, steps=20, qkv="bf16",
                 mean_rank=6, rank_cap=49, n_dense=5, seed=78)
    _run_steps(Workload(cfg), cfg.W + 4)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,V", [("mamba2", 128), ("gdn", 128), ("gdn", 80), ("kda", 128), ("kda", 64)])
def test_fp32_qkv(kind, V):
    """The float32 q/k/v instances of every family (the headline layers use bf16)."""
    cfg = _edge_cfg(kind, V, qkv="f32")
    ranks = np.array([1, 16, 0, 17, 49, 6, 3, 0], np.int32)
    _run_steps(Workload(cfg, ranks=ranks), cfg.W + 5)



# ---------------------------------------------------------------------------
# the window's last read fused into its flush (sketchssm_decode_read_flush)
# ---------------------------------------------------------------------------
@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,B", [("c0", 2), ("c1", 20), ("c2", 20), ("c3", 37), ("c4", 37)])
def test_fused_last_read(name, B):
    wl = Workload(CONFIGS[name].with_batch(B))
    _run_steps(wl, 2 * wl.cfg.W + 3, fused=True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,V,qkv", [("mamba2", 80, "bf16"), ("gdn", 128, "bf16"), ("kda", 128, "bf16"),
                                        ("mamba2", 64, "f32"), ("gdn", 80, "f32"), ("kda", 64, "f32"),
                                        ("mamba2", 96, "bf16"), ("gdn", 112, "bf16"), ("kda", 96, "f32")])
def test_fused_last_read_rank_extremes(kind, V, qkv):
    """Map tiles beyond the first (ranks 17 .. 64) and dense heads in the fused read."""
    cfg = _edge_cfg(kind, V, cap=64, qkv=qkv)
    ranks = np.array([1, 16, 0, 17, 64, 33, 49, 0], np.int32)
    _run_steps(Workload(cfg, ranks=ranks), 2 * cfg.W + 3, fused=True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,kq", [("c1", 8), ("c4", 16)])
def test_fused_last_read_shared_keys(name, kq):
    import dataclasses
    cfg = dataclasses.replace(CONFIGS[name].with_batch(19), kq_heads=kq)
    _run_steps(Workload(cfg), cfg.W + 5, fused=True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,B", [("c1", 20), ("c3", 19), ("c4", 19)])
def test_fused_last_read_dense_baseline(name, B):
    cfg = CONFIGS[name].with_batch(B)
    wl = Workload(cfg)
    wl0 = Workload(cfg, ranks=np.zeros(cfg.H, np.int32), basis=wl.basis)
    _run_steps(wl0, cfg.W + 3, dense_baseline=True, step_source=wl, fused=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,B", [("c1", 1638), ("c3", 4095), ("c4", 4095)])
def test_fused_last_read_largest_batch(name, B):
    """Each layer at the largest batch one plan takes (B H K V just below 2^31
    elements, 8.6 GB of state; offsets past 2^32 bytes, up to 209 664 flush
    blocks): a window of reads with the last one fused into its flush, checked
    on sampled rows across the batch (inputs differ in every row, see
    ``tiled_inputs``).  Afterwards the window slots that the last two reads
    appended are read back at the sampled rows and compared bit for bit with
    those tokens, so a slot address that lands on another row shows even where
    the outputs would not."""
    cfg = CONFIGS[name].with_batch(B).with_steps(CONFIGS[name].W + 2)
    wl = Workload(cfg)
    P = 23
    small = Workload(CONFIGS[name].with_batch(P))
    fill = tiled_state_fill(small, cfg.B)

    items = _sample_items(wl) + [(b, h) for b in (P, 2 * P + 1, cfg.B // 2, cfg.B - 2)
                                 for h in (0, cfg.H // 2, cfg.H - 1)]
    items = sorted(set(items))
    _log(f"  {name} at B={cfg.B}: {len(items)} sampled items")
    src = TiledRows(small, cfg.B)
    r = _run_steps(wl, cfg.steps, items=items, fused=True, step_source=src, fill_state=fill)
    _check_appended_slots(r, src, cfg.steps)


def _check_appended_slots(r, src, steps):
    """Window slots of the steps after the last flush, at the run's items,
    bitwise against the tokens of those steps."""
    W = r.cfg.W
    first = (steps - 1) // W * W  # first step of the open window
    bi, hi = torch.as_tensor(r.bi), torch.as_tensor(r.hi)
    lay = r.lay
    for t in range(first, steps):
        slot = t - first
        st = src.step(t)
        for key, buf in (("k", lay.kbuf), ("v", lay.vbuf)):
            got = buf[slot][hi, bi].cpu().view(torch.int16).numpy()
            want = st[key + "_bits"][r.bi, r.hi].view(np.int16)
            assert np.array_equal(got, want), f"window {key} slot {slot}"
        got = lay.abuf[slot][hi, bi].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), st["a"][r.bi, r.hi].view(np.uint32)), f"window decay slot {slot}"
        if lay.bbuf is not None:
            got = lay.bbuf[slot][hi, bi].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), st["beta"][r.bi, r.hi].view(np.uint32)), f"window beta slot {slot}"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c1", "c4"])
def test_fused_last_read_full_size_sampled(name):
    cfg = CONFIGS[name].with_steps(CONFIGS[name].W + 2)
    wl = Workload(cfg)
    _run_steps(wl, cfg.steps, items=_sample_items(wl), fused=True)
