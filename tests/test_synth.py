"""The seeded input generator: known answers, determinism, distributions."""
import numpy as np
import pytest

import synth
from synth.topology import chain, product_order_tree
from synth.workloads import ALL, TINY_F32, plant, step_inputs, weights


def test_philox_known_answers():
    # Known-answer vectors published with the Philox4x32-10 definition
    # (Salmon et al., SC'11, Random123 distribution): counter, key -> output.
    kat = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, want in kat:
        assert tuple(int(x) for x in synth.philox4x32_10(ctr, key)) == want


def test_normal_moments_and_determinism():
    a = synth.normal(7, 3, (400_000,), 1.0, "f32")
    b = synth.normal(7, 3, (400_000,), 1.0, "f32")
    assert np.array_equal(a, b)
    assert abs(a.mean()) < 5e-3 and abs(a.std() - 1.0) < 5e-3
    c = synth.normal(7, 4, (400_000,), 1.0, "f32")
    assert not np.array_equal(a, c)
    # any window regenerates the same elements
    w = synth.normal(7, 3, (1001,), 1.0, "f32", first=12345)
    assert np.array_equal(w, a[12345:13346])


def test_bf16_is_rne_of_f32():
    f = synth.normal(11, 5, (100_000,), 0.3, "f32")
    bb = synth.normal(11, 5, (100_000,), 0.3, "bf16")
    assert np.array_equal(bb, synth.f32_to_bf16(f))
    back = synth.bf16_to_f32(bb)
    assert np.max(np.abs(back - f) / np.abs(f)) <= 2.0 ** -8


def test_randint_range():
    r = synth.randint(3, 9, 50_000, 1024, 4096)
    assert r.min() >= 1024 and r.max() <= 4096
    assert abs(r.mean() - 2560) < 20


def test_topology_levels():
    t16 = product_order_tree((4, 2, 2, 1), 16)
    assert t16.level_counts() == [1, 3, 4, 4, 4]
    assert list(t16.paths) == [(), (0,), (1,), (2,), (0, 0), (0, 1), (1, 0), (2, 0), (0, 0, 0), (0, 0, 1),
                               (0, 1, 0), (1, 0, 0), (0, 0, 0, 0), (0, 0, 1, 0), (0, 1, 0, 0), (1, 0, 0, 0)]
    t64 = product_order_tree((10, 4, 2, 1), 64)
    assert t64.level_counts() == [1, 8, 16, 21, 18]
    ch = chain(4)
    assert ch.parent == (-1, 0, 1, 2, 3) and ch.rank == (0, 0, 0, 0, 0)
    for t in (t16, t64, ch):
        s = set(t.paths)
        for i, p in enumerate(t.paths):
            assert p[:-1] in s or p == ()  # prefix-closed
            if i:
                assert t.parent[i] < i  # parents come first
                assert t.paths[t.parent[i]] == p[:-1] and t.rank[i] == p[-1]
        # siblings take distinct ranks, so their tokens are distinct list entries
        for p in range(t.n):
            ranks = [t.rank[c] for c in range(t.n) if t.parent[c] == p]
            assert len(ranks) == len(set(ranks))


def test_workload_shapes():
    wl = TINY_F32
    w = weights(wl, 1)
    assert w["W"].shape == (4, 256, 256) and w["U"].shape == (4, 4096, 256) and not w["b"].any()
    s = step_inputs(wl, 1)
    assert s["Kc"].shape == (1, 2, 128 + 16, 64) and s["logits"].shape == (1, 16, 4096)
    b8 = ALL["70b_b8"]
    assert b8.M == 512 and b8.Lcap == 4096 + 64
    assert ALL["hydra_b4"].din == 2 * 4096


def test_plant_reaches_every_depth():
    topo = product_order_tree((4, 2, 2, 1), 16)
    B, N, V = 64, 16, 512
    rng = np.random.default_rng(0)
    logits = rng.standard_normal((B, N, V)).astype(np.float32)
    tok = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        tok[b] = rng.choice(V, N, replace=False)
    before = logits.copy()
    plant(logits, topo, tok, (1.0, 1.0, 1.0, 1.0), seed=3)
    # with a = 1 every planted child is its parent's unique argmax, on a root-to-leaf path
    changed_rows = np.argwhere(np.any(before != logits, axis=2))
    assert len(changed_rows) == 4 * B
