"""The calibration-file loader on synthetic files of the documented layout
(the real file is not available here): a basis of shape (layers, groups,
rows, K) found by name or as the only 4-D tensor, layer ids, and rejection of
files the safe loader refuses or whose basis has the wrong shape."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rank_state_read_amd.calibration import CalibrationError, load_calibration


def _save(tmp_path, obj, name="calibration.pt"):
    p = tmp_path / name
    torch.save(obj, p)
    return str(p)


def test_loads_named_basis_and_layer_ids(tmp_path):
    om = torch.randn(3, 8, 79, 128)
    p = _save(tmp_path, {"omega": om, "layer_ids": torch.tensor([1, 4, 9]), "scores": torch.randn(3, 128)})
    c = load_calibration(p)
    assert c["omega"].shape == (3, 8, 79, 128) and c["omega"].dtype == np.float32
    assert np.array_equal(c["omega"], om.numpy())
    assert c["layer_ids"] == [1, 4, 9] and c["groups"] == 8 and c["rows"] == 79


def test_finds_the_only_4d_tensor(tmp_path):
    p = _save(tmp_path, {"sketch_basis": torch.randn(2, 4, 10, 128), "ranks": torch.ones(2, 32)})
    c = load_calibration(p)
    assert c["omega"].shape == (2, 4, 10, 128) and c["layer_ids"] == [0, 1]


@pytest.mark.parametrize("obj", [
    {"omega": torch.randn(2, 8, 79, 64)},            # K mismatch
    {"omega": torch.randn(8, 79, 128)},               # not 4-D
    {"a": torch.randn(2, 8, 79, 128), "b": torch.randn(2, 8, 79, 128)},  # ambiguous
    {"omega": torch.randn(2, 8, 79, 128), "layer_ids": [1]},             # wrong id count
])
def test_rejects_bad_layouts(tmp_path, obj):
    with pytest.raises(CalibrationError):
        load_calibration(_save(tmp_path, obj))


class _Custom:
    """An arbitrary object: unpickling it would need code from this module."""


def test_rejects_files_needing_code_execution(tmp_path):
    p = _save(tmp_path, {"omega": torch.randn(1, 1, 2, 128), "obj": _Custom()})
    with pytest.raises(CalibrationError):
        load_calibration(p)
