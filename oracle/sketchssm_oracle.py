"""CPU oracle for the SketchSSM decode path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or constant generators); both only consume the seeded inputs of
the ``workloads`` package.

Plain float64 numpy, written for a reader to check against the method by eye:

* The recurrent state is always written in full; in the stretch between two
  exact flushes, reads go to a small low-rank summary of it, not to the state
  ("SketchSSM" package page, opening paragraph).
* A state update is the only time the full state is read; it keeps the
  state's products with a basis chosen offline (the sketch), and each decode
  step after it forms the output from those stored rows, weighted by numbers
  taken from the query, with no access to the state ("SketchSSM: Write to the
  Full State, Read from a Compact Sketch", Abstract).
* Keys and values are held back over a window of W tokens between flushes
  (same Abstract, which credits ReplaySSM with the idea; W = 16 in the
  Nemotron Nano 9B v2 calibration card, "Contents" table).
* Heads may be assigned a dense fallback instead of a rank ("SketchSSM"
  package page, "Make a calibration for your model", allocate stage); such
  heads read the full state.

Transitions (the three layer families named in the Abstract):
  Mamba-2  M = a I                          (scalar decay, no erase)
  GDN      M = alpha (I - beta k k^T)       (scalar decay + delta-rule erase)
  KDA      M = (I - beta k k^T) diag(alpha) (per-channel decay, then erase)
and the state update is S_t = M_t S_{t-1} + beta_t k_t v_t^T (beta = 1 for
Mamba-2), the exact output y_t = S_t^T q_t.

The sketch read of a head with rank r, basis rows Omega_r (r x K) and
coefficient map F_r (r x K), at window position j after the last flush S_0:
  q~_j  = M_1^T ... M_j^T q_j                         (query carried back)
  intra = y_exact - S_0^T q~_j                         (buffered tokens' part)
  y^    = Z^T (F_r q~_j) + intra,   Z = Omega_r S_0    (the sketch)
Dense heads output y_exact.  After the W-th read the window is flushed:
S_0 <- S, Z <- Omega_r S_0.

Two evaluation modes, which the tests require to agree to 1e-12:
  * ``ItemOracle``: one (b, h) item, transitions as explicit K x K matrices and
    an explicit product P_j = M_j ... M_1.
  * ``BatchOracle``: many items at once, matrix-free transitions, with the
    window-only state Hs (so intra = Hs^T q) and the coefficient carrier
    Q = P F_r^T (so F_r q~ = Q^T q).  This is what the parity tests use at
    size.

Parity unpinned: ``plan``'s frame order and bucket rule are this project's
own (the pages define neither), so they are pinned only against a hand-worked
example of that rule and against the library's independent planner, not
against the pages; and the pages print no worked example of y, so absolute
outputs are pinned through the exact special cases and closed forms instead.

Readings where the pages are silent are listed in the project's design notes;
the ones this file depends on: token j is read against the last flush with
itself already applied (read, then flush after the W-th read); Z is formed from
the initial state before the first read; KDA applies its decay before the
erase; the plan's frame/bucket/order rule below is this project's own (the
pages name frames and rank tables but do not define their order).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

KINDS = ("mamba2", "gdn", "kda")


# ----------------------------------------------------------------------------
# plan: frames, offsets, buckets, order (integer work)
# ----------------------------------------------------------------------------
def plan(rank: Sequence[int], group: Sequence[int], G: int, K: int,
         basis_rows: int, rank_cap: int) -> Dict[str, object]:
    """Frames and launch order derived from a per-head rank table.

    On the calibration card, a head's rank and the order of the frames are
    obtained from the calibration for whatever mean rank is asked for
    ("SketchSSM calibration: Nemotron Nano 9B v2", opening paragraph and
    "Verified mean ranks").  The
    pages do not define the order, so this rule is ours:

    * a frame is one (group, rank) coefficient map; frames are the distinct
      (group, rank) pairs of the sketch heads, sorted by group then rank;
    * frame_index[h] is the head's frame (-1 for a dense head);
    * frame_row_off is the running sum of the frames' ranks;
    * z_row_off is the running sum of the heads' ranks (a dense head has no Z);
    * bucket[h] = 0 for a dense head, else 1 + (r - 1) // 8;
    * order lists the heads: dense first, then buckets from high to low, head
      index ascending within a bucket.

    Parity unpinned by the pages (the rule is ours; see the module header).
    """
    rank = [int(x) for x in rank]
    group = [int(x) for x in group]
    H = len(rank)
    if len(group) != H:
        raise ValueError("rank and group differ in length")
    rmax = min(rank_cap, basis_rows, K)
    for h in range(H):
        if not (0 <= group[h] < G):
            raise ValueError(f"group[{h}] = {group[h]} out of range")
        if rank[h] != 0 and not (1 <= rank[h] <= rmax):
            raise ValueError(f"rank[{h}] = {rank[h]} out of range")
    frames = sorted({(group[h], rank[h]) for h in range(H) if rank[h] > 0})
    where = {f: i for i, f in enumerate(frames)}
    frame_index = [where[(group[h], rank[h])] if rank[h] > 0 else -1 for h in range(H)]
    frame_row_off = [0]
    for (_, r) in frames:
        frame_row_off.append(frame_row_off[-1] + r)
    z_row_off = [0]
    for h in range(H):
        z_row_off.append(z_row_off[-1] + rank[h])
    bucket = [0 if rank[h] == 0 else 1 + (rank[h] - 1) // 8 for h in range(H)]
    order = sorted(range(H), key=lambda h: (bucket[h] != 0, -bucket[h], h))
    return {
        "frames": frames,
        "frame_index": np.array(frame_index, dtype=np.int32),
        "frame_row_off": np.array(frame_row_off, dtype=np.int32),
        "z_row_off": np.array(z_row_off, dtype=np.int32),
        "bucket": np.array(bucket, dtype=np.int32),
        "order": np.array(order, dtype=np.int32),
        "n_frames": len(frames),
    }


# ----------------------------------------------------------------------------
# per-token transition, explicit
# ----------------------------------------------------------------------------
def transition(kind: str, a, beta, k) -> np.ndarray:
    """M_t as an explicit K x K float64 matrix."""
    k = np.asarray(k, dtype=np.float64)
    K = k.shape[0]
    eye = np.eye(K)
    if kind == "mamba2":
        return float(a) * eye
    erase = eye - float(beta) * np.outer(k, k)
    if kind == "gdn":
        return float(a) * erase
    if kind == "kda":
        return erase @ np.diag(np.asarray(a, dtype=np.float64))
    raise ValueError(kind)


def write_weight(kind: str, beta) -> float:
    return 1.0 if kind == "mamba2" else float(beta)


class ItemOracle:
    """One (b, h) item with explicit transition matrices.

    ``omega`` (r x K) and ``fmap`` (r x K) are None for a dense head.
    """

    def __init__(self, kind: str, W: int, S_init, omega=None, fmap=None):
        self.kind = kind
        self.W = W
        self.S = np.array(S_init, dtype=np.float64)
        self.K, self.V = self.S.shape
        self.dense = omega is None
        self.omega = None if self.dense else np.asarray(omega, dtype=np.float64)
        self.fmap = None if self.dense else np.asarray(fmap, dtype=np.float64)
        self._flush_state()

    def _flush_state(self):
        self.S0 = self.S.copy()
        self.P = np.eye(self.K)
        self.j = 0
        self.Z = None if self.dense else self.omega @ self.S0

    def read(self, q, k, v, a, beta=None):
        """Apply token j+1 and return (y_sketch_or_dense, y_exact)."""
        q = np.asarray(q, dtype=np.float64)
        M = transition(self.kind, a, beta, k)
        bw = write_weight(self.kind, beta)
        self.S = M @ self.S + bw * np.outer(np.asarray(k, np.float64), np.asarray(v, np.float64))
        self.P = M @ self.P
        self.j += 1
        y_exact = self.S.T @ q
        if self.dense:
            return y_exact.copy(), y_exact
        qt = self.P.T @ q
        intra = y_exact - self.S0.T @ qt
        c = self.fmap @ qt
        return self.Z.T @ c + intra, y_exact

    def flush(self):
        """Close the window: S_0 <- S, Z <- Omega_r S_0, transition product reset."""
        self._flush_state()


# ----------------------------------------------------------------------------
# many items at once, matrix-free
# ----------------------------------------------------------------------------
def _apply_transition(kind: str, X: np.ndarray, a: np.ndarray, beta: Optional[np.ndarray],
                      k: np.ndarray) -> np.ndarray:
    """M_t X for a batch: X [n, K, C], a [n] or [n, K], beta [n], k [n, K]."""
    if kind == "mamba2":
        return a[:, None, None] * X
    if kind == "gdn":
        kx = np.einsum("nk,nkc->nc", k, X)
        return a[:, None, None] * (X - beta[:, None, None] * k[:, :, None] * kx[:, None, :])
    if kind == "kda":
        DX = a[:, :, None] * X
        kx = np.einsum("nk,nkc->nc", k, DX)
        return DX - beta[:, None, None] * k[:, :, None] * kx[:, None, :]
    raise ValueError(kind)


class BatchOracle:
    """Items i = 0..n-1, each with its own state, rank, basis rows and map.

    S_init: [n, K, V].  omega / fmap: per item (r_i x K) arrays or None for a
    dense item.  Sketch quantities are zero-padded to the largest rank, which
    leaves Z^T c unchanged.

    ``traffic`` counts the bytes of stored fp32 state and sketch that the
    method moves, at the points where this class uses them: a sketch item's
    output is formed from its r_i x V sketch rows (Z read), a dense item's from
    the K x V state at the last flush (S read); a flush reads and writes the
    state once and writes the sketch (the Abstract of "SketchSSM: Write to the
    Full State, Read from a Compact Sketch": the state is read once per update,
    decode steps read only the sketch).  The initial sketch reads the state
    once and writes Z.  Window tokens and query-side data are not state and
    are not counted.
    """

    def __init__(self, kind: str, W: int, S_init: np.ndarray,
                 omega: List[Optional[np.ndarray]], fmap: List[Optional[np.ndarray]]):
        self.kind = kind
        self.W = W
        self.S = np.array(S_init, dtype=np.float64)
        n, K, V = self.S.shape
        self.n, self.K, self.V = n, K, V
        self.dense = np.array([om is None for om in omega], dtype=bool)
        self.rank = np.array([0 if om is None else om.shape[0] for om in omega], dtype=np.int64)
        self.R = max([0] + [om.shape[0] for om in omega if om is not None])
        R = max(self.R, 1)
        self.omega = np.zeros((n, R, K))
        self.fmap = np.zeros((n, R, K))
        for i in range(n):
            if omega[i] is not None:
                r = omega[i].shape[0]
                self.omega[i, :r] = omega[i]
                self.fmap[i, :r] = fmap[i]
        self.traffic = {"S_read": 0, "S_write": 0, "Z_read": 0, "Z_write": 0}
        self._flush_state(initial=True)

    def _count_flush(self, initial: bool):
        kv = 4 * self.K * self.V
        sketch = ~self.dense
        # the initial sketch only needs the sketch items' states
        self.traffic["S_read"] += kv * (int(sketch.sum()) if initial else self.n)
        if not initial:
            self.traffic["S_write"] += kv * self.n
        self.traffic["Z_write"] += 4 * self.V * int(self.rank[sketch].sum())

    def _flush_state(self, initial: bool = False):
        self._count_flush(initial)
        self.S0 = self.S.copy()
        self.Hs = np.zeros_like(self.S)                       # window-only state
        self.Q = np.transpose(self.fmap, (0, 2, 1)).copy()    # P F_r^T, P = I
        self.Z = np.einsum("nrk,nkv->nrv", self.omega, self.S0)
        self.j = 0

    def read(self, q, k, v, a, beta=None):
        """Apply one token to every item; return (y [n, V], y_exact [n, V])."""
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        a = np.asarray(a, np.float64)
        bw = np.ones(self.n) if self.kind == "mamba2" else np.asarray(beta, np.float64)
        be = None if self.kind == "mamba2" else bw
        write = bw[:, None, None] * k[:, :, None] * v[:, None, :]
        self.S = _apply_transition(self.kind, self.S, a, be, k) + write
        self.Hs = _apply_transition(self.kind, self.Hs, a, be, k) + write
        self.Q = _apply_transition(self.kind, self.Q, a, be, k)
        self.j += 1
        y_exact = np.einsum("nkv,nk->nv", self.S, q)
        c = np.einsum("nkr,nk->nr", self.Q, q)
        intra = np.einsum("nkv,nk->nv", self.Hs, q)
        y = np.einsum("nrv,nr->nv", self.Z, c) + intra
        y[self.dense] = y_exact[self.dense]
        self.traffic["Z_read"] += 4 * self.V * int(self.rank[~self.dense].sum())
        self.traffic["S_read"] += 4 * self.K * self.V * int(self.dense.sum())
        return y, y_exact

    def flush(self):
        self._flush_state()


# ----------------------------------------------------------------------------
# driving a workload
# ----------------------------------------------------------------------------
def items_oracle(wl, items: Sequence[tuple], S_init: Optional[np.ndarray] = None) -> BatchOracle:
    """BatchOracle over the listed (b, h) items of a ``workloads.Workload``."""
    cfg = wl.cfg
    if S_init is None:
        S_init = np.stack([wl.state_item(b, h) for (b, h) in items])
    omega, fmap = [], []
    for (b, h) in items:
        r = int(wl.ranks[h])
        if r == 0:
            omega.append(None)
            fmap.append(None)
        else:
            g = int(wl.groups[h])
            omega.append(wl.basis[g, :r, :].astype(np.float64))
            fmap.append(wl.fmap(g, r).astype(np.float64))
    return BatchOracle(cfg.kind, cfg.W, S_init, omega, fmap)


def gather_items(step: dict, items: Sequence[tuple]) -> dict:
    """Pick the (b, h) items out of full-batch step inputs.  When q and k have
    fewer heads than v, head h uses key/query head h // (H / Hk)."""
    bi = np.array([b for b, _ in items])
    hi = np.array([h for _, h in items])
    H = step["v"].shape[1]
    out = {}
    for key in ("q", "k", "v", "a", "beta"):
        x = step.get(key)
        if x is None:
            out[key] = None
        elif key in ("q", "k") and x.shape[1] != H:
            out[key] = x[bi, hi // (H // x.shape[1])]
        else:
            out[key] = x[bi, hi]
    return out
