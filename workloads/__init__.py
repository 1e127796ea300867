"""Seeded synthetic inputs for the SketchSSM decode path.

This module only *draws inputs*: configurations, the group-shared bases, the
synthetic per-head rank tables that stand in for a calibration, the coefficient
maps that a calibration would ship with them, the initial state and the
per-token q/k/v/decay/beta streams.  It holds none of the arithmetic of the
decode path itself (no recurrence, no sketch, no read), so the CPU oracle and
the HIP library can both consume it without sharing any of that arithmetic.

Randomness is counter based: every array is a stream of uniforms from numpy's
Philox4x64-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
SC'11) keyed by (seed, stream id, step), turned into normals by Box-Muller.
Normal number ``e`` of a stream uses uniforms ``2e`` and ``2e+1``, so any slice
of any array (one (b, h) item, one step) can be regenerated on its own without
drawing the rest.  Arrays indexed ``[b, h, ...]`` are laid out so that a
workload with a smaller batch is an exact prefix of the full one.

The shapes and value distributions follow the workloads that the SketchSSM
pages describe (the Nemotron-Nano-9B-v2 calibration card on the
"SketchSSM calibration: Nemotron Nano 9B v2" page: 128 heads, K=128, V=80,
8 basis groups of a 79x128 basis, window 16, rank cap 49, and its table of
verified mean ranks for the dense-head fractions).  The pages' accuracy suites
and model weights are not used; these synthetic draws stand in for them.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import numpy as np

KINDS = ("mamba2", "gdn", "kda")

# stream ids (second half of the Philox key); per-step streams put the step in
# the low 32 bits of the key
_ST_BASIS = 1
_ST_STATE = 2
_ST_RANKS = 3
_ST_U = 16
_ST_N = 17
_ST_K = 18
_ST_V = 19
_ST_DECAY = 20
_ST_BETA = 21


@dataclass(frozen=True)
class Config:
    """One synthetic layer workload."""

    name: str
    kind: str  # "mamba2" | "gdn" | "kda"
    B: int
    H: int
    K: int
    V: int
    G: int  # basis groups; heads are grouped contiguously, H/G per group
    W: int
    steps: int
    qkv: str  # "f32" | "bf16"
    mean_rank: float
    rank_cap: int
    n_dense: int
    seed: int
    basis_rows: int = 79
    fixed_rank: Optional[int] = None  # every sketch head gets this rank
    kq_heads: Optional[int] = None  # q/k heads, each shared by H / kq_heads heads (None: one per head)
    query_noise: float = 0.05
    state_std: float = 0.02
    decay_scale: float = 0.1

    def with_batch(self, B: int) -> "Config":
        return dataclasses.replace(self, B=B)

    def with_steps(self, steps: int) -> "Config":
        return dataclasses.replace(self, steps=steps)

    @property
    def heads_per_group(self) -> int:
        return self.H // self.G

    @property
    def Hk(self) -> int:
        """Key/query heads (H unless keys and queries are shared)."""
        return self.kq_heads or self.H

    @property
    def per_channel_decay(self) -> bool:
        return self.kind == "kda"

    @property
    def has_beta(self) -> bool:
        return self.kind in ("gdn", "kda")


# c0: tiny Mamba-2 layer; c1: Nemotron-Nano-9B-v2 Mamba-2 layer (batch 256,
# mean rank 6, 1% dense); c2: same layer at mean rank 21 with the 775/3456
# dense fraction; c3: Gated-DeltaNet layer; c4: KDA layer (per-channel decay,
# mean rank 10, 7% dense).
CONFIGS: Dict[str, Config] = {
    "c0": Config("c0", "mamba2", B=2, H=8, K=128, V=80, G=1, W=16, steps=64,
                 qkv="f32", mean_rank=6, rank_cap=49, n_dense=0, seed=1000,
                 fixed_rank=6),
    "c1": Config("c1", "mamba2", B=256, H=128, K=128, V=80, G=8, W=16, steps=512,
                 qkv="bf16", mean_rank=6, rank_cap=49,
                 n_dense=int(round(0.01 * 128)), seed=1001),
    "c2": Config("c2", "mamba2", B=512, H=128, K=128, V=80, G=8, W=16, steps=512,
                 qkv="bf16", mean_rank=21, rank_cap=49,
                 n_dense=int(round(775 / 3456 * 128)), seed=1002),
    "c3": Config("c3", "gdn", B=256, H=32, K=128, V=128, G=4, W=16, steps=512,
                 qkv="bf16", mean_rank=6, rank_cap=49, n_dense=0, seed=1003),
    "c4": Config("c4", "kda", B=512, H=32, K=128, V=128, G=4, W=16, steps=1024,
                 qkv="bf16", mean_rank=10, rank_cap=49,
                 n_dense=int(round(0.07 * 32)), seed=1004),
}


# ----------------------------------------------------------------------------
# counter-based draws
# ----------------------------------------------------------------------------
def _key(seed: int, stream: int, step: int = 0) -> np.ndarray:
    return np.array([np.uint64(seed) & np.uint64(0xFFFFFFFFFFFFFFFF),
                     (np.uint64(stream) << np.uint64(32)) | np.uint64(step)],
                    dtype=np.uint64)


def uniforms(seed: int, stream: int, step: int, start: int, count: int) -> np.ndarray:
    """Uniforms number ``start .. start+count-1`` of stream (seed, stream, step)."""
    if count <= 0:
        return np.zeros(0, dtype=np.float64)
    block, skip = divmod(int(start), 4)
    bg = np.random.Philox(key=_key(seed, stream, step),
                          counter=np.array([block, 0, 0, 0], dtype=np.uint64))
    out = np.random.Generator(bg).random(skip + int(count))
    return out[skip:]


def normals(seed: int, stream: int, step: int, start: int, count: int) -> np.ndarray:
    """Standard normals number ``start .. start+count-1`` (Box-Muller, fp64)."""
    u = uniforms(seed, stream, step, 2 * int(start), 2 * int(count))
    u0 = u[0::2]
    u1 = u[1::2]
    return np.sqrt(-2.0 * np.log1p(-u0)) * np.cos(2.0 * np.pi * u1)


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even)."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------
# synthetic calibration stand-ins
# ----------------------------------------------------------------------------
def make_basis(cfg: Config) -> np.ndarray:
    """[G, basis_rows, K] float32, each group's rows orthonormal.

    QR of a seeded K x basis_rows Gaussian; column signs are flipped so that
    diag(R) > 0, which makes the basis independent of the LAPACK in use.
    """
    out = np.empty((cfg.G, cfg.basis_rows, cfg.K), dtype=np.float32)
    for g in range(cfg.G):
        a = normals(cfg.seed, _ST_BASIS, g, 0, cfg.K * cfg.basis_rows).reshape(cfg.K, cfg.basis_rows)
        q, r = np.linalg.qr(a)
        sgn = np.sign(np.diag(r))
        sgn[sgn == 0] = 1.0
        q = q * sgn[None, :]
        out[g] = q.T.astype(np.float32)
    return out


def make_ranks(cfg: Config) -> np.ndarray:
    """Per-head rank table, int32 [H]; 0 marks a dense-fallback head.

    Dense heads: a seeded random subset of n_dense heads.  Sketch heads: a
    geometric draw with mean ``mean_rank`` capped at ``rank_cap``, rescaled so
    that the ranks sum to round(mean_rank * n_sketch) (floors first, then the
    remaining units by descending fractional part, lower head first on ties;
    any excess is taken from the largest ranks, higher head first on ties).
    """
    H = cfg.H
    if cfg.fixed_rank is not None:
        r = np.full(H, cfg.fixed_rank, dtype=np.int32)
        return r
    rng = np.random.Generator(np.random.Philox(key=_key(cfg.seed, _ST_RANKS)))
    dense = np.sort(rng.permutation(H)[: cfg.n_dense])
    is_dense = np.zeros(H, dtype=bool)
    is_dense[dense] = True
    heads = np.nonzero(~is_dense)[0]
    n = len(heads)
    cap = cfg.rank_cap
    ranks = np.zeros(H, dtype=np.int64)
    if n == 0:
        return ranks.astype(np.int32)
    mu = float(cfg.mean_rank)
    g = np.minimum(rng.geometric(1.0 / mu, size=n), cap).astype(np.float64)
    T = int(round(mu * n))
    x = g * T / g.sum()
    r = np.clip(np.floor(x), 1, cap).astype(np.int64)
    frac = x - np.floor(x)
    rem = T - int(r.sum())
    while rem > 0:
        cand = [i for i in np.argsort(-frac, kind="stable") if r[i] < cap]
        if not cand:
            break
        for i in cand:
            if rem == 0:
                break
            r[i] += 1
            rem -= 1
    while rem < 0:
        # largest rank first, higher head on ties
        order = sorted(range(n), key=lambda i: (-r[i], -i))
        took = False
        for i in order:
            if rem == 0:
                break
            if r[i] > 1:
                r[i] -= 1
                rem += 1
                took = True
        if not took:
            break
    ranks[heads] = r
    return ranks.astype(np.int32)


def make_groups(cfg: Config) -> np.ndarray:
    return (np.arange(cfg.H) // cfg.heads_per_group).astype(np.int32)


def coefficient_map(basis: np.ndarray, g: int, r: int) -> np.ndarray:
    """F_r = pinv(Omega_r)^T for the first r rows of group g's basis; float32 [r, K].

    This is what a calibration ships per (group, rank) frame; for orthonormal
    rows it equals Omega_r up to rounding.
    """
    om = basis[g, :r, :].astype(np.float64)
    return np.linalg.pinv(om).T.astype(np.float32)


# ----------------------------------------------------------------------------
# the workload
# ----------------------------------------------------------------------------
class Workload:
    """All inputs of one configuration, drawn lazily and deterministically."""

    def __init__(self, cfg: Config, ranks: Optional[np.ndarray] = None,
                 basis: Optional[np.ndarray] = None):
        assert cfg.kind in KINDS
        assert cfg.H % cfg.G == 0
        assert cfg.H % cfg.Hk == 0
        self.cfg = cfg
        self.basis = make_basis(cfg) if basis is None else np.asarray(basis, dtype=np.float32)
        self.ranks = make_ranks(cfg) if ranks is None else np.asarray(ranks, dtype=np.int32)
        self.groups = make_groups(cfg)
        self._fmaps: Dict[Tuple[int, int], np.ndarray] = {}

    # -- calibration stand-ins -------------------------------------------
    def fmap(self, g: int, r: int) -> np.ndarray:
        key = (int(g), int(r))
        if key not in self._fmaps:
            self._fmaps[key] = coefficient_map(self.basis, g, r)
        return self._fmaps[key]

    def head_fmap(self, h: int) -> Optional[np.ndarray]:
        r = int(self.ranks[h])
        return None if r == 0 else self.fmap(int(self.groups[h]), r)

    # -- initial state -----------------------------------------------------
    def state_item(self, b: int, h: int) -> np.ndarray:
        c = self.cfg
        n = c.K * c.V
        x = normals(c.seed, _ST_STATE, 0, (b * c.H + h) * n, n) * c.state_std
        return x.reshape(c.K, c.V).astype(np.float32)

    def state_batch(self, b: int) -> np.ndarray:
        """S_init[b] as float32 [H, K, V]."""
        c = self.cfg
        n = c.H * c.K * c.V
        x = normals(c.seed, _ST_STATE, 0, b * n, n) * c.state_std
        return x.reshape(c.H, c.K, c.V).astype(np.float32)

    def state(self) -> np.ndarray:
        c = self.cfg
        out = np.empty((c.B, c.H, c.K, c.V), dtype=np.float32)
        for b in range(c.B):
            out[b] = self.state_batch(b)
        return out

    # -- per-token inputs --------------------------------------------------
    def _cast_qkv(self, x64: np.ndarray):
        x32 = x64.astype(np.float32)
        if self.cfg.qkv == "f32":
            return x32, None
        bits = to_bf16_bits(x32)
        return bf16_bits_to_f32(bits), bits

    def _tokens(self, t: int, b0: int, b1: int, heads: np.ndarray) -> dict:
        """Inputs of step t for batch rows b0..b1-1 and the given heads.  q and k
        are per key/query head: for the key heads of the given heads, in order."""
        c = self.cfg
        R = c.rank_cap
        nb = b1 - b0
        Hk = c.Hk
        share = c.H // Hk
        kheads = np.unique(np.asarray(heads) // share)

        def draw(stream, width, total, idx):
            out = np.empty((nb, len(idx), width), dtype=np.float64)
            if len(idx) == total and np.array_equal(idx, np.arange(total)):
                out[:] = normals(c.seed, stream, t, b0 * total * width, nb * total * width).reshape(nb, total, width)
                return out
            for bi in range(nb):
                for j, h in enumerate(idx):
                    out[bi, j] = normals(c.seed, stream, t, ((b0 + bi) * total + int(h)) * width, width)
            return out

        u = draw(_ST_U, R, Hk, kheads)
        n = draw(_ST_N, c.K, Hk, kheads)
        kk = draw(_ST_K, c.K, Hk, kheads)
        vv = draw(_ST_V, c.V, c.H, heads)
        dx = draw(_ST_DECAY, c.K if c.per_channel_decay else 1, c.H, heads)
        bx = draw(_ST_BETA, 1, c.H, heads) if c.has_beta else None

        # a query lies near the span of the basis rows its heads read: with a
        # shared query, the largest rank among the sketch heads that share it
        q = np.empty((nb, len(kheads), c.K), dtype=np.float64)
        for j, kh in enumerate(kheads):
            members = [h for h in range(int(kh) * share, (int(kh) + 1) * share) if self.ranks[h] > 0]
            if not members:
                q[:, j, :] = n[:, j, :]
            else:
                r = max(int(self.ranks[h]) for h in members)
                om = self.basis[int(self.groups[members[0]]), :r, :].astype(np.float64)
                q[:, j, :] = u[:, j, :r] @ om + c.query_noise * n[:, j, :]
        kk = kk / np.linalg.norm(kk, axis=-1, keepdims=True)
        a = np.exp(-_softplus(dx) * c.decay_scale)
        if not c.per_channel_decay:
            a = a[..., 0]
        out = {}
        out["q"], out["q_bits"] = self._cast_qkv(q)
        out["k"], out["k_bits"] = self._cast_qkv(kk)
        out["v"], out["v_bits"] = self._cast_qkv(vv)
        out["a"] = a.astype(np.float32)
        out["beta"] = None if bx is None else _sigmoid(bx[..., 0]).astype(np.float32)
        return out

    def step(self, t: int) -> dict:
        """Inputs of step t for the whole batch: arrays [B, H, ...] (q, k: [B, Hk, K])."""
        return self._tokens(t, 0, self.cfg.B, np.arange(self.cfg.H))

    def step_item(self, t: int, b: int, h: int) -> dict:
        """Inputs of step t for one (b, h) item (same values as ``step(t)``)."""
        d = self._tokens(t, b, b + 1, np.array([h]))
        return {k: (None if v is None else v[0, 0]) for k, v in d.items()}


def describe(cfg: Config) -> str:
    return (f"{cfg.name}: {cfg.kind} B={cfg.B} H={cfg.H} K={cfg.K} V={cfg.V} G={cfg.G} "
            f"W={cfg.W} steps={cfg.steps} qkv={cfg.qkv} mean_rank={cfg.mean_rank} "
            f"dense={cfg.n_dense}" + (f" kq_heads={cfg.kq_heads}" if cfg.kq_heads else ""))
