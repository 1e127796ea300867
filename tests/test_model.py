"""The multi-layer decode loop's host logic, on stand-in layers (no GPU): every
token visits every layer in order, positions cycle through the window, the last
position goes to the fused read-and-flush call, and inconsistent set-ups are
refused."""
import pytest

pytest.importorskip("torch")

from rank_state_read_amd.model import SketchModel  # noqa: E402


class _Layer:
    def __init__(self, name, W=16, log=None):
        self.name, self.W, self.log = name, W, log

    def flush(self, n, stream=None):
        self.log.append((self.name, "flush", n))

    def read(self, pos, q, k, v, a, beta=None, stream=None):
        self.log.append((self.name, "read", pos, q))
        return f"y-{self.name}"

    def read_flush(self, q, k, v, a, beta=None, stream=None):
        self.log.append((self.name, "read_flush", q))
        return f"y-{self.name}"


def test_token_loop_and_window_cycle():
    log = []
    layers = [_Layer(i, W=4, log=log) for i in range(3)]
    m = SketchModel(layers, layer_ids=[3, 7, 11])
    m.start()
    assert log == [(0, "flush", 0), (1, "flush", 0), (2, "flush", 0)] and m.pos == 0
    log.clear()
    for t in range(9):
        toks = [{"q": (t, i), "k": None, "v": None, "a": None} for i in range(3)]
        ys = m.decode_step(toks)
        assert ys == ["y-0", "y-1", "y-2"]
    expect = []
    for t in range(9):
        for i in range(3):
            if t % 4 == 3:
                expect.append((i, "read_flush", (t, i)))
            else:
                expect.append((i, "read", t % 4, (t, i)))
    assert log == expect and m.pos == 9 % 4


def test_refuses_inconsistent_setups():
    log = []
    with pytest.raises(ValueError):
        SketchModel([])
    with pytest.raises(ValueError):
        SketchModel([_Layer(0, 16, log), _Layer(1, 8, log)])
    with pytest.raises(ValueError):
        SketchModel([_Layer(0, 16, log)], layer_ids=[1, 2])
    m = SketchModel([_Layer(0, 16, log), _Layer(1, 16, log)])
    with pytest.raises(ValueError):
        m.decode_step([{"q": 0, "k": 0, "v": 0, "a": 0}])
