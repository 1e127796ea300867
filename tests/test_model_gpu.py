"""A multi-layer decode loop with each layer's basis from a calibration file.

The Nemotron Nano 9B v2 calibration card ("SketchSSM calibration: Nemotron
Nano 9B v2 (BF16 weights)", "Contents") describes a file read with
``torch.load(..., weights_only=True)`` that holds one group-shared basis per
recurrent layer, float32 of shape (layers, 8, 79, 128), with the model index of
each layer in ``layer_ids``.  The real file is not available here, so a
synthetic file of that layout is written (orthonormal rows per layer and group,
each layer drawn from its own seed, plus a stand-in for the allocation scores)
and read back by the library's loader.  Three Nano-shaped Mamba-2 layers,
each with its own rank table, state, sketch and window and the basis of its
file entry, then decode two windows and a few tokens through
``SketchModel`` (every layer per token, the window's last read fused into the
flush), and every layer's y, S and Z is compared with its own oracle."""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from workloads import CONFIGS, Workload, make_basis  # noqa: E402
from parity_run import PrefetchedSteps, Run, _log, _sample_items  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_state_read_amd import binding
    binding.lib()


def _layer_cfg(i, B, kind="c1"):
    return dataclasses.replace(CONFIGS[kind].with_batch(B), seed=CONFIGS[kind].seed + 100 * (i + 1),
                               name=f"{kind}-layer{i}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("n_layers,B", [(3, 19)])
def test_multi_layer_decode_with_calibration_file(tmp_path, n_layers, B):
    from rank_state_read_amd.calibration import load_calibration
    from rank_state_read_amd.model import SketchModel

    cfgs = [_layer_cfg(i, B) for i in range(n_layers)]
    layer_ids = [2 * i + 1 for i in range(n_layers)]          # model indices of the recurrent layers
    omega = np.stack([make_basis(c) for c in cfgs])            # (layers, 8, 79, 128)
    path = tmp_path / "calibration.pt"
    torch.save({"omega": torch.from_numpy(omega), "layer_ids": torch.tensor(layer_ids),
                "scores": torch.rand(n_layers, cfgs[0].H, cfgs[0].basis_rows)}, path)
    cal = load_calibration(str(path), K=cfgs[0].K)
    assert cal["omega"].shape == (n_layers, 8, 79, 128) and cal["layer_ids"] == layer_ids

    wls = [Workload(c, basis=cal["omega"][i]) for i, c in enumerate(cfgs)]
    # the layers differ in everything a layer owns
    assert not np.array_equal(wls[0].ranks, wls[1].ranks)
    assert not np.array_equal(wls[0].basis, wls[1].basis)
    W = cfgs[0].W
    steps = 2 * W + 3
    runs = [Run(wl, items=_sample_items(wl), step_source=PrefetchedSteps(wl, steps, workers=4))
            for wl in wls]
    model = SketchModel([r.lay for r in runs], layer_ids=cal["layer_ids"])
    model.start()
    torch.cuda.synchronize()
    for r in runs:
        r.check_Z()
    for t in range(steps):
        sts = [r.src.step(t) for r in runs]
        devs = [r.lay.upload_step(st) for st in sts]
        pos = model.pos
        assert pos == t % W
        ys = model.decode_step(devs)
        for r, st, y in zip(runs, sts, ys):
            r.finish(st, y, pos)
    for i, r in enumerate(runs):
        assert len(r.history) == 2
        _log(f"  layer {cal['layer_ids'][i]}: {len(r.items)} items, max errors {r.max_err}")
