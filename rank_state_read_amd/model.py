"""A model's recurrent layers decoded one token at a time.

The Nemotron Nano 9B v2 calibration card ("SketchSSM calibration: Nemotron
Nano 9B v2 (BF16 weights)", "Contents") lists 27 recurrent layers, each with
its own group-shared basis (the basis array is (27, 8, 79, 128), with the model
layer index of each entry in ``layer_ids``).  Every such layer keeps its own
state cache, sketch and window; one decode token passes through all of them in
turn.  ``SketchModel`` holds those layers (``SketchLayer`` objects, one per
recurrent layer, all with the same window length) and runs that loop over the
C entry points: at window position 0 .. W-2 each layer's read, at W-1 each
layer's last read fused into its flush.  All layers share one window phase,
since every layer sees every token.

Only the recurrent part of a layer is here: the projections that produce a
layer's q, k, v, decay and beta from the previous layer's output are not part of
the decode path this library implements, so the caller supplies each layer's
token inputs.  No arithmetic happens in this module.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import torch

from .layer import SketchLayer


class SketchModel:
    def __init__(self, layers: Sequence[SketchLayer], layer_ids: Optional[Sequence[int]] = None):
        if not layers:
            raise ValueError("a model needs at least one recurrent layer")
        W = layers[0].W
        if any(L.W != W for L in layers):
            raise ValueError("all layers must share one window length")
        self.layers: List[SketchLayer] = list(layers)
        self.layer_ids = list(range(len(layers))) if layer_ids is None else [int(i) for i in layer_ids]
        if len(self.layer_ids) != len(self.layers):
            raise ValueError("one layer id per layer")
        self.W = W
        self.pos = 0

    def start(self, stream=None):
        """Form every layer's first sketch from its current state (after a
        prefill) and restart the window at position 0."""
        for L in self.layers:
            L.flush(0, stream=stream)
        self.pos = 0

    def decode_step(self, tokens: Sequence[Dict[str, Optional[torch.Tensor]]], stream=None) -> List[torch.Tensor]:
        """One token through every layer.  ``tokens[i]`` holds layer i's device
        inputs (``q``, ``k``, ``v``, ``a`` and, for the delta rule, ``beta``);
        returns the layers' output buffers (each layer's ``y``, overwritten by
        the next step)."""
        if len(tokens) != len(self.layers):
            raise ValueError("one token input per layer")
        last = self.pos == self.W - 1
        out = []
        for L, d in zip(self.layers, tokens):
            if last:
                out.append(L.read_flush(d["q"], d["k"], d["v"], d["a"], d.get("beta"), stream=stream))
            else:
                out.append(L.read(self.pos, d["q"], d["k"], d["v"], d["a"], d.get("beta"), stream=stream))
        self.pos = (self.pos + 1) % self.W
        return out
