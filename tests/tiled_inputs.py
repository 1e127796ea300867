"""Inputs for a large batch drawn cheaply from a small one (test helper).

Row b of the large batch takes the tokens of row b % P of the small workload,
with q and v scaled by a power of two that changes every P rows (exact in
bf16), and an initial state that is row b % P's scaled by 1 + b / 2048.  Every
row's outputs are then its own, while only P rows are ever drawn."""
import numpy as np


class TiledRows:
    """Step source (``step(t)`` as ``workloads.Workload.step``) for B rows."""

    def __init__(self, small, B):
        self.small = small
        self.P = small.cfg.B
        self.idx = np.arange(B) % self.P
        self.scale = 2.0 ** ((np.arange(B) // self.P) % 5 - 2)

    def step(self, t):
        from workloads import to_bf16_bits
        st = self.small.step(t)
        out = {}
        for key, val in st.items():
            if val is None or key.endswith("_bits"):
                continue
            x = val[self.idx]
            if key in ("q", "v"):
                x = (x * self.scale.reshape((-1,) + (1,) * (x.ndim - 1))).astype(val.dtype)
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
