"""The seeded input generator: determinism, slicing, shapes and distributions."""
import json
import os

import numpy as np

from workloads import (CONFIGS, Workload, bf16_bits_to_f32, make_ranks, normals,
                       to_bf16_bits)


def test_counter_slices_match_whole_stream():
    whole = normals(5, 18, 3, 0, 1000)
    for start, cnt in [(0, 1), (1, 7), (13, 100), (999, 1)]:
        np.testing.assert_array_equal(normals(5, 18, 3, start, cnt), whole[start:start + cnt])
    assert not np.array_equal(normals(5, 18, 4, 0, 10), whole[:10])
    assert not np.array_equal(normals(6, 18, 3, 0, 10), whole[:10])


def test_normals_are_standard():
    x = normals(1, 17, 0, 0, 200_000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -3.14159, 0.0, 1e-30], np.float32)
    got = bf16_bits_to_f32(to_bf16_bits(x))
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert got[1] == 1.0
    assert got[2] == np.float32(1.0078125)
    assert got[3] == np.float32(1.0078125)
    assert np.all(np.abs(got - x) <= np.abs(x) * 2.0 ** -8)


def test_smaller_batch_is_prefix():
    big = Workload(CONFIGS["c3"].with_batch(3))
    small = Workload(CONFIGS["c3"].with_batch(2))
    a, b = big.step(5), small.step(5)
    for k in ("q", "k", "v", "a", "beta"):
        np.testing.assert_array_equal(a[k][:2], b[k])
    np.testing.assert_array_equal(big.state_batch(1), small.state_batch(1))


def test_step_item_matches_step():
    wl = Workload(CONFIGS["c4"].with_batch(2))
    st = wl.step(2)
    for (b, h) in [(0, 0), (1, 31), (1, 7)]:
        it = wl.step_item(2, b, h)
        for k in ("q", "k", "v", "a", "beta"):
            np.testing.assert_array_equal(st[k][b, h], it[k])


def test_value_distributions():
    wl = Workload(CONFIGS["c4"].with_batch(4))
    st = wl.step(0)
    nk = np.linalg.norm(st["k"].astype(np.float64), axis=-1)
    assert np.all(np.abs(nk - 1) < 5e-3)          # unit keys, up to bf16 rounding
    assert st["a"].shape == (4, 32, 128)          # KDA: per-channel decay
    assert np.all((st["a"] > 0) & (st["a"] < 1))
    assert np.all((st["beta"] > 0) & (st["beta"] < 1))
    # bf16 values: the low 16 bits of each float32 are zero
    assert np.all(st["q"].view(np.uint32) & 0xFFFF == 0)
    c0 = Workload(CONFIGS["c0"]).step(0)
    assert c0["q_bits"] is None and c0["q"].dtype == np.float32
    s = wl.state_batch(0)
    assert abs(s.std() - 0.02) < 5e-4


def test_basis_rows_orthonormal():
    wl = Workload(CONFIGS["c1"].with_batch(1))
    for g in range(wl.cfg.G):
        om = wl.basis[g].astype(np.float64)
        np.testing.assert_allclose(om @ om.T, np.eye(79), atol=1e-6)
        F = wl.fmap(g, 6).astype(np.float64)
        np.testing.assert_allclose(F @ om[:6].T, np.eye(6), atol=1e-6)


def test_rank_tables_hit_the_budget():
    for name, cfg in CONFIGS.items():
        r = make_ranks(cfg)
        assert r.shape == (cfg.H,)
        assert (r == 0).sum() == cfg.n_dense
        sk = r[r > 0]
        assert sk.min() >= 1 and sk.max() <= cfg.rank_cap
        assert sk.sum() == round(cfg.mean_rank * len(sk))
        np.testing.assert_array_equal(r, make_ranks(cfg))


def test_nano_layer_matches_calibration_card(golden_dir):
    with open(os.path.join(golden_dir, "nano_card.json")) as f:
        card = json.load(f)
    c1 = CONFIGS["c1"]
    assert (c1.H, c1.K, c1.V, c1.G, c1.W, c1.rank_cap) == (
        card["state_heads_per_layer"], card["K"], card["V"], card["basis_groups_per_layer"],
        card["window"], card["rank_cap"])
    assert c1.basis_rows == card["basis_shape"][2] and c1.K == card["basis_shape"][3]
    assert c1.kind == "mamba2" and card["erase_factor"] is False
    tab = {row["mean_rank"]: row for row in card["verified_mean_ranks"]}
    total = 27 * 128
    assert tab[21]["dense"] + tab[21]["sketch"] == total
    # dense fractions of the Nano-shaped workloads follow the card's table
    assert CONFIGS["c2"].n_dense == round(tab[21]["dense"] / total * 128)
    assert abs(tab[6]["dense"] / total - 0.01) < 0.002 and CONFIGS["c1"].n_dense == 1
    assert abs(tab[10]["dense"] / total - 0.07) < 0.01


def test_shared_keys_gather_to_their_heads():
    """With keys and queries shared by groups of heads, the oracle's per-item
    gather picks each head's key/query head and matches the single-item draw."""
    import dataclasses
    from oracle import gather_items
    cfg = dataclasses.replace(CONFIGS["c1"].with_batch(3), kq_heads=8)
    wl = Workload(cfg)
    st = wl.step(4)
    assert st["q"].shape == (3, 8, 128) and st["k"].shape == (3, 8, 128) and st["v"].shape == (3, 128, 80)
    items = [(0, 0), (1, 15), (1, 16), (2, 127), (2, 64)]
    g = gather_items(st, items)
    for i, (b, h) in enumerate(items):
        one = wl.step_item(4, b, h)
        for key in ("q", "k", "v", "a"):
            assert np.array_equal(g[key][i], one[key]), (key, b, h)
        assert np.array_equal(g["k"][i], st["k"][b, h // 16])


def test_tiled_rows_for_large_batches():
    """The large-batch inputs of the largest-batch GPU tests: row b takes row
    b % P of a small draw with heads rotated by s = b // P, the key's channels
    rotated by (s // Hk) mod K, decays and betas scaled by 2^-((s // H) mod 8)
    and q, v by 2^(((s // Hx) + s) mod 8 - 3); the bf16 bits agree with the
    values, and no row repeats another at the largest batches."""
    from tiled_inputs import TiledRows
    P = 23
    for name, B, rows in (("c1", 130, (0, 22, 23, 77, 129)), ("c3", 4095, (0, 24, 736, 2944, 4094))):
        small = Workload(CONFIGS[name].with_batch(P))
        tr = TiledRows(small, B)
        st, s0 = tr.step(3), small.step(3)
        H, K = small.cfg.H, small.cfg.K
        for key in ("q", "k", "v"):
            assert np.array_equal(bf16_bits_to_f32(st[key + "_bits"]), st[key]), key
        for b in rows:
            s = b // P
            for h in (0, 5, H - 1):
                hh = (h + s) % H
                rot = (s // H) % K
                for c in (0, 1, 77, K - 1):
                    assert st["k"][b, h, c] == s0["k"][b % P, hh, (c + rot) % K]
                assert st["a"][b, h] == np.float32(s0["a"][b % P, hh] * 2.0 ** -((s // H) % 8))
                e = ((s // H) + s) % 8 - 3
                assert np.array_equal(st["q"][b, h], (s0["q"][b % P, hh] * 2.0 ** e).astype(np.float32))
                assert np.array_equal(st["v"][b, h], (s0["v"][b % P, hh] * 2.0 ** e).astype(np.float32))
                if st["beta"] is not None:
                    assert st["beta"][b, h] == np.float32(s0["beta"][b % P, hh] * 2.0 ** -((s // H) % 8))
        for key in ("q", "k", "v", "a"):
            assert len(np.unique(st[key].reshape(B, -1), axis=0)) == B, (name, key)
