"""Inputs for a large batch drawn cheaply from a small one (test helper).

Row b of the large batch takes the tokens of row b % P of the small workload,
transformed by exact operations keyed on s = b // P, so that rows a multiple of
P apart do not repeat one another:
  * every per-head input takes head (h + s) mod Hx of its row (Hx = Hk for q
    and k, H for v, decay and beta);
  * the key's channels, and KDA's per-channel decays, are rotated by
    (s // Hx) mod K (a rotation keeps a key's norm exactly), so (head
    rotation, channel rotation) repeats only after Hx K blocks of P rows;
  * scalar decays and betas are scaled by 2^-((s // H) mod 8), so they repeat
    only after 8 H blocks;
  * q and v are scaled by 2^(((s // Hx) + s) mod 8 - 3) (exact in bf16), which
    changes from block to block and repeats only after 8 Hx blocks.
With P = 23 no row of any input repeats within 8 * 32 * 23 = 5888 rows, more
than the largest batch a plan takes for any layer here.  The initial state of
row b is row b % P's scaled by 1 + b / 2048, different in every row.  Every
row's outputs are then its own, while only P rows are ever drawn."""
import numpy as np


class TiledRows:
    """Step source (``step(t)`` as ``workloads.Workload.step``) for B rows."""

    def __init__(self, small, B):
        self.small = small
        self.P = small.cfg.B
        self.B = B
        rows = np.arange(B)
        self.idx = rows % self.P
        self.s = rows // self.P

    def _rotate_heads(self, x):
        Hx = x.shape[1]
        hidx = (np.arange(Hx)[None, :] + self.s[:, None]) % Hx
        return x[np.arange(self.B)[:, None], hidx]

    def _rotate_channels(self, x):
        Hx, K = x.shape[1], x.shape[-1]
        rot = (self.s // Hx) % K
        cidx = (np.arange(K)[None, :] + rot[:, None]) % K
        return x[np.arange(self.B)[:, None, None], np.arange(Hx)[None, :, None], cidx[:, None, :]]

    def step(self, t):
        from workloads import to_bf16_bits
        st = self.small.step(t)
        out = {}
        for key, val in st.items():
            if val is None or key.endswith("_bits"):
                continue
            x = self._rotate_heads(val[self.idx])
            if key == "k" or (key == "a" and x.ndim == 3):
                x = self._rotate_channels(x)
            elif key in ("a", "beta"):
                x = x * 2.0 ** (-((self.s // x.shape[1]) % 8))[:, None]
            if key in ("q", "v"):
                e = ((self.s // x.shape[1]) + self.s) % 8 - 3
                x = x * (2.0 ** e)[:, None, None]
            x = np.ascontiguousarray(x, dtype=val.dtype)
            out[key] = x
            if st.get(key + "_bits") is not None:
                out[key + "_bits"] = to_bf16_bits(x.astype(np.float32))
        out.setdefault("beta", None)
        return out


def tiled_state_fill(small, B):
    """fill(S): writes the tiled initial state into the device tensor S [B,H,K,V]."""
    import torch
    P = small.cfg.B
    base = torch.from_numpy(np.stack([small.state_batch(b) for b in range(P)])).cuda()

    def fill(S):
        for b in range(B):
            S[b].copy_(base[b % P] * (1.0 + b / 2048.0))
    return fill
