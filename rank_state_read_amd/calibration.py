"""Reading a SketchSSM calibration file (host side, no arithmetic of the path).

The calibration card for Nemotron Nano 9B v2 (page "SketchSSM calibration:
Nemotron Nano 9B v2 (BF16 weights)", "Contents") describes ``calibration.pt``:
a file that ``torch.load(..., weights_only=True)`` reads, holding the
group-shared basis ``omega`` as float32 of shape (layers, groups, rows, K) --
(27, 8, 79, 128) for that model -- the model layer index of each stored layer
(``layer_ids``), and the allocation scores from which rank tables are derived.
The key names beyond these are documented in a guide that is not available
here, so the loader looks for the basis by name (``omega`` or ``basis``) and
otherwise for the one 4-D float32 tensor in the file; the allocation scores
are not used (the rank allocation rule is not part of the decode path).

Nothing is executed from the file: it is opened with ``weights_only=True`` and
rejected if that loader refuses it.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np


class CalibrationError(ValueError):
    pass


def _find_basis(obj) -> Optional[object]:
    if isinstance(obj, dict):
        for key in ("omega", "basis"):
            if key in obj:
                return obj[key]
        cands = [v for v in obj.values() if hasattr(v, "dim") and v.dim() == 4]
        if len(cands) == 1:
            return cands[0]
    return None


def load_calibration(path: str, K: int = 128) -> Dict[str, object]:
    """Basis (layers, groups, rows, K) float32 and the layer ids of a calibration file."""
    import torch

    try:
        obj = torch.load(path, map_location="cpu", weights_only=True)
    except Exception as e:  # the safe loader refused the file
        raise CalibrationError(f"{path}: not loadable with weights_only=True ({e})") from e
    basis = _find_basis(obj)
    if basis is None:
        raise CalibrationError(f"{path}: no basis tensor (expected key 'omega' or 'basis')")
    if basis.dim() != 4 or basis.shape[-1] != K:
        raise CalibrationError(f"{path}: basis shape {tuple(basis.shape)} is not (layers, groups, rows, {K})")
    omega = basis.detach().to(torch.float32).contiguous().numpy()
    if not np.isfinite(omega).all():
        raise CalibrationError(f"{path}: basis has non-finite entries")
    L = omega.shape[0]
    ids = obj.get("layer_ids") if isinstance(obj, dict) else None
    layer_ids: List[int] = list(range(L)) if ids is None else [int(x) for x in list(ids)]
    if len(layer_ids) != L:
        raise CalibrationError(f"{path}: {len(layer_ids)} layer ids for {L} layers")
    return {"omega": omega, "layer_ids": layer_ids, "groups": omega.shape[1], "rows": omega.shape[2]}
