"""Caller-side device buffers of one recurrent layer, allocated with torch.

The library allocates nothing; this helper owns the state cache, the sketch,
the window, the packed frames and the output of one layer and forwards to the
C entry points.  It does no arithmetic of the decode path: it only allocates,
copies inputs in and lays out the frames array in the plan's frame order.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np
import torch

from . import binding as _b


def _to_device(x, dtype, device):
    if isinstance(x, torch.Tensor):
        return x.to(device=device, dtype=dtype).contiguous()
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dtype).contiguous()


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """A bfloat16 device tensor holding the given raw 16-bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


class SketchLayer:
    """One layer's buffers for ``sketchssm_flush`` / ``sketchssm_decode_read``.

    rank, group : int32 [H] (rank 0 = dense fallback)
    basis       : float32 [G, basis_rows, K]
    fmap        : callable (group, rank) -> float32 [rank, K] coefficient map
    S_init      : float32 [B, H, K, V] (numpy or tensor), or None to leave S empty
    """

    def __init__(self, *, B: int, H: int, K: int, V: int, W: int, G: int, basis_rows: int,
                 rank_cap: int, kind: str, qkv: str, rank, group, basis,
                 fmap: Optional[Callable] = None, S_init=None, device="cuda", kq_heads: int = 0,
                 order=None):
        self.kind, self.qkv = kind, qkv
        self.B, self.H, self.K, self.V, self.W = B, H, K, V, W
        self.Hk = int(kq_heads) if kq_heads else H
        self.device = torch.device(device)
        self.shape = _shape(B, H, K, V, W, G, basis_rows, rank_cap, kind, qkv, kq_heads)
        self.plan = _plan(self.shape, rank, group, order)
        self.layout = self.plan.export()
        dev = self.device
        self.S = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
        if S_init is not None:
            self.S.copy_(_to_device(S_init, torch.float32, dev))
        nz = self.plan.z_elems
        self.Z = torch.zeros(max(nz, 4), dtype=torch.float32, device=dev) if nz else None
        self.basis = _to_device(basis, torch.float32, dev)
        nf = self.plan.frame_elems
        self.frames = None
        if nf:
            packed = np.zeros(nf, dtype=np.float32)
            off = self.layout["frame_row_off"]
            for f, (g, r) in enumerate(self.layout["frames"]):
                packed[off[f] * K:(off[f] + r) * K] = np.asarray(fmap(g, r), np.float32).reshape(-1)
            self.frames = _to_device(packed, torch.float32, dev)
        qdt = torch.bfloat16 if qkv == "bf16" else torch.float32
        self.qdtype = qdt
        # the window: slot-major [W][H][B][...] (keys [W][Hk][B][K]), so one
        # decode step appends one contiguous slab and a block's batch rows are
        # adjacent
        self.kbuf = torch.zeros((W, self.Hk, B, K), dtype=qdt, device=dev)
        self.vbuf = torch.zeros((W, H, B, V), dtype=qdt, device=dev)
        self.abuf = torch.zeros((W, H, B, K) if kind == "kda" else (W, H, B), dtype=torch.float32, device=dev)
        self.bbuf = torch.zeros((W, H, B), dtype=torch.float32, device=dev) if kind != "mamba2" else None
        self.y = torch.empty((B, H, V), dtype=torch.float32, device=dev)

    # -- inputs ------------------------------------------------------------
    def upload_step(self, st: dict) -> dict:
        """Copy one step's inputs (the ``workloads`` dict layout) to the device."""
        dev = self.device
        out = {}
        for key in ("q", "k", "v"):
            if self.qkv == "bf16":
                out[key] = bf16_tensor(st[key + "_bits"], dev)
            else:
                out[key] = _to_device(st[key], torch.float32, dev)
        out["a"] = _to_device(st["a"], torch.float32, dev)
        out["beta"] = None if st.get("beta") is None else _to_device(st["beta"], torch.float32, dev)
        return out

    # -- the entry points -----------------------------------------------------
    def flush(self, n_tokens: int, stream=None):
        _b.sketchssm_flush(self.plan, self.S, self.Z, self.basis, self.kbuf, self.vbuf, self.abuf,
                          self.bbuf, n_tokens, stream)

    def read(self, pos: int, q, k, v, a, beta=None, y=None, stream=None) -> torch.Tensor:
        y = self.y if y is None else y
        _b.sketchssm_decode_read(self.plan, self.S, self.Z, self.frames, q, k, v, a, beta, self.kbuf,
                                self.vbuf, self.abuf, self.bbuf, pos, y, stream)
        return y

    def read_flush(self, q, k, v, a, beta=None, y=None, stream=None, plan=None) -> torch.Tensor:
        """The window's last read and its flush in one pass (``plan``: e.g. an
        all-dense plan for the full-state-read baseline)."""
        y = self.y if y is None else y
        pl = self.plan if plan is None else plan
        _b.sketchssm_decode_read_flush(pl, self.S, self.Z if plan is None else None,
                                      self.frames if plan is None else None,
                                      self.basis if plan is None else None, q, k, v, a, beta, self.kbuf,
                                      self.vbuf, self.abuf, self.bbuf, y, stream)
        return y

    def dense_read(self, pos: int, q, k, v, a, beta=None, y=None, stream=None) -> torch.Tensor:
        y = self.y if y is None else y
        _b.sketchssm_dense_read(self.shape, self.S, q, k, v, a, beta, self.kbuf, self.vbuf, self.abuf,
                               self.bbuf, pos, y, stream)
        return y

    def read_seq(self, pos, q, k, v, a, beta=None, y=None, stream=None) -> torch.Tensor:
        """Decode read with a window position per sequence (device int32 [B]; -1 idles a row)."""
        y = self.y if y is None else y
        _b.sketchssm_decode_read_seq(self.plan, self.S, self.Z, self.frames, q, k, v, a, beta, self.kbuf,
                                    self.vbuf, self.abuf, self.bbuf, pos, y, stream)
        return y

    def flush_seq(self, seqs, n_tokens, stream=None):
        """Flush the listed sequences (device int32 rows and per-row token counts)."""
        _b.sketchssm_flush_seq(self.plan, self.S, self.Z, self.basis, self.kbuf, self.vbuf, self.abuf,
                              self.bbuf, seqs, n_tokens, int(seqs.numel()), stream)

    def rmw_step(self, q, k, v, a, beta=None, y=None, stream=None) -> torch.Tensor:
        """Standard per-token decode on this layer's state (no window, no sketch)."""
        y = self.y if y is None else y
        _b.sketchssm_rmw_step(self.shape, self.S, q, k, v, a, beta, y, stream)
        return y

    # -- views ---------------------------------------------------------------
    def z_item(self, b: int, h: int) -> Optional[torch.Tensor]:
        """The (rank x V) sketch rows of item (b, h), or None for a dense head."""
        r = int(self.plan.rank[h])
        if r == 0:
            return None
        z0 = int(self.layout["z_row_off"][h])
        start = (z0 * self.B + b * r) * self.V
        return self.Z[start:start + r * self.V].view(r, self.V)

    def z_items(self, items) -> list:
        return [self.z_item(b, h) for (b, h) in items]


def _shape(B_, H, K, V, W, G, basis_rows, rank_cap, kind, qkv, kq_heads=0):
    return _b.make_shape(B_, H, K, V, W, G, basis_rows, rank_cap, kind, qkv, kq_heads)


def _plan(shape, rank, group, order=None):
    return _b.Plan(shape, rank, group, order)


def launch_order(rank, kind: str = "bucket"):
    """A launch order for ``sketchssm_plan_create_ordered``: dense heads first
    (ascending), then the sketch heads in head order ("head"), by rank bucket
    from low to high ("low-first"), or from high to low ("bucket", the
    planner's own order)."""
    rank = np.asarray(rank, np.int64)
    dense = [h for h in range(len(rank)) if rank[h] == 0]
    sk = [h for h in range(len(rank)) if rank[h] > 0]
    bucket = {h: 1 + (int(rank[h]) - 1) // 8 for h in sk}
    if kind == "head":
        pass
    elif kind == "low-first":
        sk.sort(key=lambda h: (bucket[h], h))
    elif kind == "bucket":
        sk.sort(key=lambda h: (-bucket[h], h))
    else:
        raise ValueError(f"unknown launch order {kind!r}")
    return np.array(dense + sk, np.int32)


def layer_for_workload(wl, *, ranks=None, device="cuda", S_init=None, with_state=True,
                       order=None) -> SketchLayer:
    """A SketchLayer for a ``workloads.Workload`` (ranks may be overridden, e.g.
    all zero; ``order``: an explicit launch order, see ``launch_order``)."""
    c = wl.cfg
    rk = wl.ranks if ranks is None else np.asarray(ranks, np.int32)
    lay = SketchLayer(B=c.B, H=c.H, K=c.K, V=c.V, W=c.W, G=c.G, basis_rows=c.basis_rows,
                      rank_cap=c.rank_cap, kind=c.kind, qkv=c.qkv, rank=rk, group=wl.groups,
                      basis=wl.basis, fmap=wl.fmap, S_init=None, device=device,
                      kq_heads=c.kq_heads or 0, order=order)
    if S_init is not None:
        lay.S.copy_(_to_device(S_init, torch.float32, lay.device))
    elif with_state:
        for b in range(c.B):
            lay.S[b].copy_(torch.from_numpy(wl.state_batch(b)))
    return lay
