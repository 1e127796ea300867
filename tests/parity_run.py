"""Shared driver of the GPU parity tests: one layer on the GPU through the C
ABI beside the float64 oracle on a set of (b, h) items, every output and every
flushed state and sketch compared within 1e-4 relative per slab (max |gpu -
ref| / max |ref|; a slab is one (t, b, h) output vector, one item's K x V state
or one item's r x V sketch).  Also the item sampler used at full batch sizes and
a step source that draws a run's inputs ahead of use on host threads."""
import sys
import time
from collections import deque
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import gather_items, items_oracle

TOL = 1e-4


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _slab_err(got, ref):
    """max over slabs of max|got-ref| / max|ref|; slabs along the leading axis."""
    got = np.asarray(got, np.float64).reshape(len(ref), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((np.abs(got - ref).max(axis=1) / den).max())


class Run:
    """Drive one layer on the GPU and the oracle on a set of (b, h) items."""

    def __init__(self, wl, items=None, dense_baseline=False, step_source=None, z_error_bound=False,
                 fused=False, fill_state=None, order=None):
        from rank_state_read_amd.layer import layer_for_workload
        self.wl = wl
        c = wl.cfg
        self.cfg = c
        self.dense = dense_baseline
        self.src = step_source or wl
        # fill_state(S): writes the initial state into the device tensor instead
        # of the workload's own draw
        self.lay = layer_for_workload(wl, with_state=fill_state is None, order=order)
        if fill_state is not None:
            fill_state(self.lay.S)
        self.items = items if items is not None else [(b, h) for b in range(c.B) for h in range(c.H)]
        S0 = np.stack([self.lay.S[b, h].cpu().numpy() for (b, h) in self.items]) \
            if len(self.items) < c.B * c.H else self.lay.S.cpu().numpy().reshape(-1, c.K, c.V)
        self.orc = items_oracle(wl, self.items, S_init=S0)
        self.bi = np.array([b for b, _ in self.items])
        self.hi = np.array([h for _, h in self.items])
        self.sketch_items = [i for i, (b, h) in enumerate(self.items) if wl.ranks[h] > 0]
        self.t = 0
        self.max_err = {"y": 0.0, "S": 0.0, "Z": 0.0}
        # per closed window: (step, max y error over the window's reads, S error, Z error)
        self.history = []
        self._win_y = 0.0
        # With z_error_bound, a sketch whose rows cancel (basis rows nearly
        # orthogonal to a low-rank state, |Omega_r S| << |Omega_r| |S|) is held
        # to the fp32 forward error bound of its K-term products, (K + 2) u
        # |Omega_r| |S| (u = 2^-24), where that exceeds 1e-4 of the slab.
        self.z_error_bound = z_error_bound
        # fused: the window's last read and its flush in one call
        self.fused = fused

    def init_sketch(self):
        self.lay.flush(0)
        torch.cuda.synchronize()
        self.check_Z()

    def check_S(self):
        S = self.lay.S[torch.as_tensor(self.bi), torch.as_tensor(self.hi)].cpu().numpy()
        e = _slab_err(S, self.orc.S0)
        self.max_err["S"] = max(self.max_err["S"], e)
        assert e <= TOL, f"S after flush at t={self.t}: {e:.3e}"
        return e

    def check_Z(self):
        if not self.sketch_items:
            return 0.0
        e = 0.0
        for i in self.sketch_items:
            b, h = self.items[i]
            r = int(self.wl.ranks[h])
            g = self.lay.z_item(b, h).cpu().numpy().astype(np.float64)
            rr = self.orc.Z[i, :r]
            den = max(np.abs(rr).max(), 1e-30)
            if self.z_error_bound:
                om = np.abs(self.wl.basis[int(self.wl.groups[h]), :r].astype(np.float64))
                bound = (self.cfg.K + 2) * 2.0 ** -24 * (om @ np.abs(self.orc.S0[i])).max()
                den = max(den, bound / TOL)
            e = max(e, float(np.abs(g - rr).max() / den))
        self.max_err["Z"] = max(self.max_err["Z"], e)
        assert e <= TOL, f"Z at t={self.t}: {e:.3e}"
        return e

    def step(self, check=True):
        c = self.cfg
        st = self.src.step(self.t)
        dev = self.lay.upload_step(st)
        pos = self.t % c.W
        if self.fused and pos == c.W - 1:
            y = self.lay.read_flush(dev["q"], dev["k"], dev["v"], dev["a"], dev["beta"])
        else:
            if self.dense:
                y = self.lay.dense_read(pos, dev["q"], dev["k"], dev["v"], dev["a"], dev["beta"])
            else:
                y = self.lay.read(pos, dev["q"], dev["k"], dev["v"], dev["a"], dev["beta"])
            if pos == c.W - 1:
                self.lay.flush(c.W)
        self.finish(st, y, pos, check)

    def finish(self, st, y, pos, check=True):
        """The oracle's step on the same inputs and the comparison with the
        GPU output y (and, after the window's last read, with S and Z)."""
        c = self.cfg
        so = gather_items(st, self.items)
        yo, _ = self.orc.read(so["q"], so["k"], so["v"], so["a"], so["beta"])
        torch.cuda.synchronize()
        self.t += 1
        if check:
            yg = y[torch.as_tensor(self.bi), torch.as_tensor(self.hi)].cpu().numpy()
            e = _slab_err(yg, yo)
            self.max_err["y"] = max(self.max_err["y"], e)
            self._win_y = max(self._win_y, e)
            assert e <= TOL, f"y at t={self.t - 1} (pos {pos}): {e:.3e}"
        if self.orc.j == c.W:
            self.orc.flush()
            if check:
                eS = self.check_S()
                eZ = self.check_Z()
                self.history.append((self.t, self._win_y, eS, eZ))
            self._win_y = 0.0


def _run_steps(wl, steps, **kw):
    r = Run(wl, **kw)
    r.init_sketch()
    t0 = time.time()
    for _ in range(steps):
        r.step()
    _log(f"  {wl.cfg.name} B={wl.cfg.B} steps={steps} max errors {r.max_err} ({time.time() - t0:.1f}s)")
    return r


def _sample_items(wl):
    c = wl.cfg
    items = []
    seen = set()
    for h in range(c.H):
        r = int(wl.ranks[h])
        key = ("d", h) if r == 0 else (int(wl.groups[h]), r)
        if key in seen:
            continue
        seen.add(key)
        for b in (0, c.B - 1):
            items.append((b, h))
    rng = np.random.default_rng(c.seed)
    for _ in range(16):
        items.append((int(rng.integers(c.B)), int(rng.integers(c.H))))
    return sorted(set(items))


class PrefetchedSteps:
    """Step source for a run of n consecutive steps (``step(t)`` as
    ``workloads.Workload.step``, called for t = 0, 1, 2, ... in order) whose
    inputs are drawn up to ``ahead`` steps in advance on host threads.  The
    draws are the workload's own (counter-based, so order does not matter);
    numpy's generators and ufuncs release the interpreter lock while they run,
    so the threads overlap the drawing with the GPU and oracle work."""

    def __init__(self, source, n_steps, workers=8, ahead=24):
        self.source = source
        self.n = n_steps
        self.ahead = ahead
        self.pool = ThreadPoolExecutor(max_workers=workers)
        self.pending = deque()
        self.next_t = 0
        self.issued = 0
        for _ in range(min(ahead, n_steps)):
            self._issue()

    def _issue(self):
        self.pending.append(self.pool.submit(self.source.step, self.issued))
        self.issued += 1

    def step(self, t):
        assert t == self.next_t, f"steps must be taken in order ({t} after {self.next_t - 1})"
        out = self.pending.popleft().result()
        self.next_t += 1
        if self.issued < self.n:
            self._issue()
        if self.next_t == self.n:
            self.pool.shutdown(wait=False)
        return out
