"""The C-ABI library on the host: it loads, exports every declared symbol, its
planner matches the oracle's plan rule bit for bit, and argument errors come
back as status codes before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import plan as oracle_plan
from rank_state_read_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    syms = set()
    inc = os.path.join(ROOT, "include")
    for name in sorted(os.listdir(inc)):
        if not name.endswith(".h"):
            continue
        with open(os.path.join(inc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        syms |= set(re.findall(r"\b(sketchssm_[a-z_]+)\s*\(", text))
    return sorted(syms)


def test_library_exports_every_declared_symbol():
    syms = _declared_symbols()
    assert len(syms) >= 9
    L = B.lib()
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(B._PROTOS)


def _shape(H=8, G=2, B_=4, V=80, kind="mamba2", qkv="bf16", cap=49, rows=79, kq=0):
    return B.make_shape(B_, H, 128, V, 16, G, rows, cap, kind, qkv, kq)


def test_plan_matches_oracle_rule_bit_exact():
    rng = np.random.default_rng(11)
    for trial in range(300):
        H = int(rng.integers(1, 257))
        G = int(rng.integers(1, 9))
        cap = int(rng.integers(1, 65))
        rows = int(rng.integers(1, 80))
        rmax = min(cap, rows, 128)
        rank = rng.integers(0, rmax + 1, size=H).astype(np.int32)
        rank[rng.random(H) < rng.random()] = 0
        group = rng.integers(0, G, size=H).astype(np.int32)
        p = B.Plan(_shape(H=H, G=G, cap=cap, rows=rows), rank, group)
        got = p.export()
        want = oracle_plan(rank, group, G, 128, rows, cap)
        assert got["frames"] == [tuple(f) for f in want["frames"]]
        for key in ("frame_index", "frame_row_off", "z_row_off", "bucket", "order"):
            assert np.array_equal(got[key], want[key]), (trial, key)
        assert p.z_elems == 4 * 80 * int(rank.sum())
        assert p.frame_elems == 128 * sum(r for _, r in want["frames"])


def test_plan_hand_example_from_library(golden_dir):
    import json
    with open(os.path.join(golden_dir, "plan_small.json")) as f:
        g = json.load(f)
    p = B.Plan(_shape(H=8, G=g["G"]), np.array(g["rank"]), np.array(g["group"]))
    got = p.export()
    assert [list(x) for x in got["frames"]] == g["frames"]
    for key in ("frame_index", "frame_row_off", "z_row_off", "bucket", "order"):
        assert got[key].tolist() == g[key], key


def test_plan_with_explicit_order():
    """sketchssm_plan_create_ordered: the given order, every other table as the
    derived plan's; a non-permutation or a dense head after a sketch head is
    refused."""
    from rank_state_read_amd.layer import launch_order
    rng = np.random.default_rng(5)
    for trial in range(100):
        H = int(rng.integers(1, 257))
        G = int(rng.integers(1, 9))
        rank = rng.integers(0, 50, size=H).astype(np.int32)
        rank[rng.random(H) < 0.2] = 0
        group = rng.integers(0, G, size=H).astype(np.int32)
        sh = _shape(H=H, G=G)
        base = B.Plan(sh, rank, group).export()
        for kind in ("bucket", "head", "low-first"):
            o = launch_order(rank, kind)
            got = B.Plan(sh, rank, group, o).export()
            assert np.array_equal(got["order"], o)
            for key in ("frame_index", "frame_row_off", "z_row_off", "bucket"):
                assert np.array_equal(got[key], base[key]), (trial, kind, key)
            assert got["frames"] == base["frames"]
        # the planner's own order is the "bucket" order
        assert np.array_equal(launch_order(rank, "bucket"), base["order"])
    sh = _shape(H=4, G=1)
    rank = np.array([0, 3, 5, 0], np.int32)
    group = np.zeros(4, np.int32)
    for bad in ([0, 1, 2, 2], [0, 1, 2, 4], [0, 1, 3, 2], [1, 0, 3, 2]):
        with pytest.raises(RuntimeError, match="ESHAPE"):
            B.Plan(sh, rank, group, np.array(bad, np.int32))
    ok = B.Plan(sh, rank, group, np.array([3, 0, 2, 1], np.int32)).export()
    assert ok["order"].tolist() == [3, 0, 2, 1]


@pytest.mark.parametrize("bad", [
    dict(H=0), dict(H=257), dict(V=72), dict(V=48), dict(V=144), dict(G=0), dict(cap=65), dict(B_=0),
    dict(kq=3), dict(kq=16), dict(kq=-1),
    # one layer's state must stay below 2^31 elements: 1639 x 128 x 128 x 80 is past it
    dict(B_=1639, H=128, G=8),
])
def test_plan_rejects_bad_shapes(bad):
    kw = dict(H=8, G=2)
    kw.update(bad)
    H = max(kw["H"], 1)
    with pytest.raises(B.SketchSSMError) as e:
        B.Plan(_shape(**kw), np.ones(H, np.int32), np.zeros(H, np.int32))
    assert e.value.status == 2


def test_largest_state_is_accepted():
    """1638 sequences of the Nano layer (128 heads, 128 x 80 state): 8.0 GiB of
    state, the most one plan takes."""
    p = B.Plan(_shape(B_=1638, H=128, G=8), np.ones(128, np.int32), np.repeat(np.arange(8), 16))
    assert p.z_elems == 1638 * 80 * 128


def test_plan_rejects_bad_tables():
    for rank, group in [([50] + [1] * 7, [0] * 8), ([-1] + [1] * 7, [0] * 8),
                        ([1] * 8, [2] + [0] * 7), ([80] + [1] * 7, [0] * 8)]:
        with pytest.raises(B.SketchSSMError) as e:
            B.Plan(_shape(), np.array(rank), np.array(group))
        assert e.value.status == 2
    # rank above basis_rows
    with pytest.raises(B.SketchSSMError):
        B.Plan(_shape(rows=5), np.array([6] + [1] * 7), np.zeros(8))


def test_bad_kind_and_dtype():
    for kw in (dict(kind=3), dict(qkv=2)):
        with pytest.raises(B.SketchSSMError) as e:
            B.Plan(_shape(**kw), np.ones(8, np.int32), np.zeros(8, np.int32))
        assert e.value.status == 1


# Host-side argument checks of the launch entry points: every case below is
# rejected before any HIP call, so no device is touched.
FAKE = 1 << 20  # a 16-byte-aligned stand-in address, never dereferenced


def test_read_argument_errors():
    p = B.Plan(_shape(), np.array([0, 1, 2, 3, 4, 5, 6, 7]), np.zeros(8, np.int32))
    L = B.lib()
    args = dict(S=FAKE, Z=FAKE, frames=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, beta=None,
                kbuf=FAKE, vbuf=FAKE, abuf=FAKE, bbuf=None, pos=0, y=FAKE)

    def call(**over):
        a = dict(args)
        a.update(over)
        return L.sketchssm_decode_read(p.handle, a["S"], a["Z"], a["frames"], a["q"], a["k"], a["v"],
                                       a["a"], a["beta"], a["kbuf"], a["vbuf"], a["abuf"], a["bbuf"],
                                       a["pos"], a["y"], None)

    assert call(pos=-1) == 1
    assert call(pos=16) == 1
    assert call(q=None) == 1
    assert call(y=None) == 1
    assert call(S=None) == 1          # a dense head is present
    assert call(Z=None) == 1          # sketch heads are present
    assert call(beta=FAKE) == 1       # Mamba-2 takes no beta
    assert call(q=FAKE + 4) == 3      # misaligned
    assert L.sketchssm_decode_read(None, *([None] * 12), 0, None, None) == 1


def test_flush_argument_errors():
    sh = _shape(kind="gdn", V=128)
    p = B.Plan(sh, np.array([0, 1, 2, 3, 4, 5, 6, 7]), np.zeros(8, np.int32))
    L = B.lib()

    def call(S=FAKE, Z=FAKE, basis=FAKE, kb=FAKE, vb=FAKE, ab=FAKE, bb=FAKE, n=16):
        return L.sketchssm_flush(p.handle, S, Z, basis, kb, vb, ab, bb, n, None)

    assert call(n=-1) == 1
    assert call(n=17) == 1
    assert call(S=None) == 1
    assert call(Z=None) == 1
    assert call(bb=None) == 1         # delta rule needs beta
    assert call(basis=FAKE + 8) == 3


def test_dense_read_argument_errors():
    L = B.lib()
    bad = _shape(V=72)
    assert L.sketchssm_dense_read(ctypes.byref(bad), *([FAKE] * 5), None, FAKE, FAKE, FAKE, None, 0,
                                  FAKE, None) == 2
    ok = _shape()
    assert L.sketchssm_dense_read(ctypes.byref(ok), *([FAKE] * 5), None, FAKE, FAKE, FAKE, None, 99,
                                  FAKE, None) == 1


def test_rmw_step_argument_errors():
    L = B.lib()
    ok = _shape()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE]            # S q k v a beta y
    assert L.sketchssm_rmw_step(ctypes.byref(_shape(V=72)), *args, None) == 2
    assert L.sketchssm_rmw_step(ctypes.byref(ok), *([None] + args[1:]), None) == 1
    assert L.sketchssm_rmw_step(ctypes.byref(ok), *(args[:5] + [FAKE, FAKE]), None) == 1  # beta with Mamba-2
    gdn = _shape(kind="gdn", V=128)
    assert L.sketchssm_rmw_step(ctypes.byref(gdn), *args, None) == 1                       # GDN needs beta
    assert L.sketchssm_rmw_step(ctypes.byref(ok), *(args[:6] + [FAKE + 4]), None) == 3     # misaligned y
    assert L.sketchssm_rmw_step(None, *args, None) == 1


def test_seq_entry_points_argument_errors():
    L = B.lib()
    plan = B.Plan(_shape(), np.full(8, 6, np.int32), np.repeat(np.arange(2, dtype=np.int32), 4))
    h = plan.handle
    rd = [FAKE] * 12                                                  # S Z frames q k v a beta kbuf vbuf abuf bbuf
    rd[7] = None
    rd[11] = None                                                     # Mamba-2: no beta, no bbuf
    assert L.sketchssm_decode_read_seq(h, *rd, None, FAKE, None) == 1  # no positions
    assert L.sketchssm_decode_read_seq(None, *rd, FAKE, FAKE, None) == 1
    assert L.sketchssm_decode_read_seq(h, *rd, FAKE + 2, FAKE, None) == 3  # misaligned positions
    fl = [FAKE] * 7                                                    # S Z basis kbuf vbuf abuf bbuf
    fl[6] = None
    assert L.sketchssm_flush_seq(h, *fl, None, FAKE, 1, None) == 1     # no row list
    assert L.sketchssm_flush_seq(h, *fl, FAKE, None, 1, None) == 1     # no counts
    assert L.sketchssm_flush_seq(h, *fl, FAKE, FAKE, -1, None) == 1    # negative length
    assert L.sketchssm_flush_seq(h, *(fl[:3] + [None] + fl[4:]), FAKE, FAKE, 1, None) == 1  # window needed
    assert L.sketchssm_flush_seq(h, *fl, FAKE, FAKE, 0, None) == 0     # empty list: nothing to do
    assert L.sketchssm_flush_seq(h, *fl, FAKE + 2, FAKE, 1, None) == 3


def test_read_flush_argument_errors():
    L = B.lib()
    plan = B.Plan(_shape(), np.array([0, 1, 2, 3, 4, 5, 6, 7]), np.zeros(8, np.int32))
    h = plan.handle
    # S Z frames basis q k v a beta kbuf vbuf abuf bbuf y
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE]

    def call(**over):
        names = ["S", "Z", "frames", "basis", "q", "k", "v", "a", "beta", "kbuf", "vbuf", "abuf", "bbuf", "y"]
        a = dict(zip(names, ok))
        a.update(over)
        return L.sketchssm_decode_read_flush(h, *[a[n] for n in names], None)

    assert call(y=None) == 1
    assert call(q=None) == 1
    assert call(frames=None) == 1     # sketch heads need their maps
    assert call(beta=FAKE) == 1       # Mamba-2 takes no beta
    assert call(kbuf=None) == 1       # the window is read
    assert call(y=FAKE + 4) == 3      # misaligned
    assert L.sketchssm_decode_read_flush(None, *([None] * 14), None) == 1


def test_shared_key_heads_accepted():
    for kq in (0, 1, 2, 4, 8):
        B.Plan(_shape(kq=kq), np.full(8, 3, np.int32), np.repeat(np.arange(2, dtype=np.int32), 4))


def test_status_strings():
    for s in range(7):
        assert B.status_string(s)
    assert "unknown" in B.status_string(42)


def test_stream_probe_argument_errors():
    """The measurement probe's argument rules are checked before any launch."""
    L = B.lib()
    a16 = 1 << 20            # a 16-byte-aligned stand-in address (never dereferenced)
    probe = L.sketchssm_stream_probe
    assert probe(None, 8 * 4096, a16, 0, 8, 4, 0, None) == 1            # null source
    assert probe(a16 + 4, 8 * 4096, a16, 0, 8, 4, 0, None) == 3         # unaligned
    assert probe(a16, 8 * 4096, a16, 0, 6, 4, 0, None) == 1             # unroll not 4/8/16
    assert probe(a16, 8 * 4096 + 16, a16, 0, 8, 4, 0, None) == 2        # not whole chunks
    assert probe(a16, 8 * 4096, a16, 3 * 4096, 8, 0, 0, None) == 2      # ratio not an integer
    assert probe(a16, 16 * 4096, a16, 4096, 8, 0, 0, None) == 2         # ratio 16 > unroll 8
    assert probe(a16, 8 * 4096, a16, 0, 8, 0, 0, None) == 1             # read-only needs a bounded grid
    assert probe(a16, 8 * 4096, a16, 0, 8, -1, 0, None) == 1            # negative grid
    assert probe(a16, 8 * 4096, a16, 0, 8, 4, 2, None) == 1             # unknown flag


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """With the HIP library absent every entry point raises: there is no
    fallback path."""
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libsketchssm.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()
    with pytest.raises(RuntimeError, match="missing"):
        B.Plan(_shape(), np.zeros(8, np.int32), np.zeros(8, np.int32))
