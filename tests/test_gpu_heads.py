"""GPU parity of md_medusa_heads against the oracle (Medusa and Hydra).

Top-k lists follow the margin rule of _helpers; h' and the top-k values the
relative tolerance. Sizes span several row tiles per wave and ragged tails
(V = 5003), every activation-row grouping (M = 1, 2, 3, 5), and the full
8B- and 70B-shaped heads.
"""
import math
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from synth.topology import product_order_tree
from synth.workloads import HYDRA_B4, LLAMA8B, LLAMA70B, LLAMA70B_SHARED, TINY_F32, Workload, step_inputs, weights

from _helpers import TAU, TOL, check_topk, from_dev, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _md():
    import medusa_draft_heads_amd as md

    return md


def gpu_heads_medusa(wl: Workload, wd, h_dev, M, U_op=None, U_norms=None, W_op=None):
    import torch

    md = _md()
    K, kmax = wl.K, wl.kmax
    kind = md.MD_HEADS_MEDUSA_SHARED if wl.shared_u else md.MD_HEADS_MEDUSA
    dt = md.MD_F32 if wl.dtype == "f32" else md.MD_BF16
    idx = torch.empty(M, K, kmax, dtype=torch.int32, device="cuda")
    val = torch.empty(M, K, kmax, dtype=torch.float32, device="cuda")
    hres = torch.empty(K, M, wl.d, dtype=torch.float32, device="cuda")
    ws = torch.empty(md.md_heads_workspace_bytes(kind, dt, M, wl.d, wl.V, K, kmax), dtype=torch.uint8, device="cuda")
    md.md_medusa_heads(kind, dt, M, wl.d, wl.V, K, wl.topk, 0, None, h_dev, wd["W"], wd["b"], wd["U"], None, None,
                       None, idx, val, hres, ws, U_op=U_op, U_norms=U_norms, W_op=W_op)
    torch.cuda.synchronize()
    return from_dev(idx), from_dev(val), from_dev(hres)


def compare_medusa(wl, gi, gv, gh, ref, label=""):
    tau, tol = TAU[wl.dtype], TOL[wl.dtype]
    ties = 0
    for k in range(wl.K):
        lg = ref.get("logits")
        ties += check_topk(gi[:, k], gv[:, k], ref["idx"][:, k], ref["val"][:, k], ref["margin"][:, k], wl.topk[k],
                           tau, tol, logits_of=(lambda r, ii, k=k: lg[r, k, ii]) if lg is not None else None)
        assert np.all(gi[:, k, wl.topk[k]:] == -1)
    err = rel_err(gh, ref["hres"])
    assert err <= tol, "%s h' relative error %.3g" % (label, err)
    print("%s: h' rel err %.2e, near-tie lists %d of %d" % (label, err, ties, gi.shape[0] * wl.K))
    return ties


SMALL_BF16 = Workload("small bf16: d=512 V=5003 K=3", "medusa", B=1, d=512, V=5003, K=3, dtype="bf16",
                      topk=(6, 3, 1), N=10, Hq=4, Hkv=1, hd=64, L=10)


@pytest.mark.parametrize("wl,M", [(TINY_F32, 1), (replace(TINY_F32, V=1111, bias_zero=False), 4),
                                  (SMALL_BF16, 1), (SMALL_BF16, 2), (SMALL_BF16, 3), (SMALL_BF16, 5),
                                  (replace(SMALL_BF16, topk=(16, 1, 16)), 2),
                                  (replace(SMALL_BF16, d=256, V=777), 1), (replace(SMALL_BF16, d=64, V=300), 1),
                                  (replace(SMALL_BF16, topk=(16, 1, 16)), 1)])
def test_heads_medusa_small(wl, M):
    """One bf16 row runs the single fused launch (residual blocks, projections, top-k and merge;
    d = 64 and 256 leave h' smaller than the block's list area in LDS), more rows and float32 the
    separate kernels."""
    seed = 1000 + M
    w = weights(wl, seed)
    h = synth.normal(seed, 77, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi, gv, gh, ref, label="%s M=%d" % (wl.name, M))
    # run twice: bit-identical
    gi2, gv2, gh2 = gpu_heads_medusa(wl, wd, to_dev(h), M)
    assert np.array_equal(gi, gi2) and np.array_equal(gv.view(np.uint32), gv2.view(np.uint32))


@pytest.mark.parametrize("wl", [SMALL_BF16, replace(SMALL_BF16, d=256, V=777, topk=(16, 1, 4))],
                         ids=["d=512", "d=256"])
def test_heads_fused_give_up_paths(wl):
    """The single-launch kernel's bounded waits, forced to give up from the host (md_set_wait_limits):
    with no polls for its group's h', every block computes its head's h' alone from W and h, and the
    lists, values and h' equal the normal launch's bit for bit (and the oracle's); with no polls for
    the lists, each head's merging block gives up and writes -1 indices and -inf values."""
    md = _md()
    seed = 4500 + wl.d
    w = weights(wl, seed)
    h = synth.normal(seed, 87, (1, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    assert md.md_heads_fused(md.MD_HEADS_MEDUSA, md.MD_BF16, 1, wl.d, wl.K)
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), 1)
    try:
        md.md_set_wait_limits(0, -1)
        gi2, gv2, gh2 = gpu_heads_medusa(wl, wd, to_dev(h), 1)
        md.md_set_wait_limits(-1, 0)
        gi3, gv3, _ = gpu_heads_medusa(wl, wd, to_dev(h), 1)
    finally:
        md.md_set_wait_limits(-1, -1)
    assert np.array_equal(gi, gi2) and np.array_equal(gv.view(np.uint32), gv2.view(np.uint32))
    assert np.array_equal(gh.view(np.uint32), gh2.view(np.uint32))
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi2, gv2, gh2, ref, label="%s, every block computing h' alone" % wl.name)
    assert np.all(gi3 == -1) and np.all(np.isneginf(gv3))
    # and the normal limits again: the normal result
    gi4, gv4, _ = gpu_heads_medusa(wl, wd, to_dev(h), 1)
    assert np.array_equal(gi, gi4) and np.array_equal(gv.view(np.uint32), gv4.view(np.uint32))


def test_heads_structured_cases():
    """W = 0, b = 0 gives h' = h; U = I (V = d) gives the sorted h itself."""
    import torch

    d, V, K = 256, 256, 2
    wl = Workload("identity", "medusa", B=1, d=d, V=V, K=K, dtype="f32", topk=(16, 5), N=1, Hq=1, Hkv=1, hd=64, L=0)
    h = synth.normal(5, 1, (3, d), 1.0, "f32")
    wd = {"W": torch.zeros(K, d, d, device="cuda"), "b": torch.zeros(K, d, device="cuda"),
          "U": torch.eye(d, device="cuda").repeat(K, 1, 1).contiguous()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), 3)
    assert np.array_equal(gh[0], h) and np.array_equal(gh[1], h)
    for m in range(3):
        ref = np.argsort(-h[m].astype(np.float64), kind="stable")
        assert np.array_equal(gi[m, 0, :16], ref[:16]) and np.array_equal(gi[m, 1, :5], ref[:5])
        assert np.array_equal(gv[m, 0, :16], h[m][ref[:16]])


@pytest.mark.parametrize("wl_name", ["8b", "70b"])
def test_heads_medusa_full_size(wl_name):
    wl = LLAMA8B if wl_name == "8b" else LLAMA70B
    w = weights(wl, 8 if wl_name == "8b" else 70)
    h = step_inputs(wl, 8 if wl_name == "8b" else 70)["h"]
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), 1)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi, gv, gh, ref, label=wl.name)
    del wd


# ---------------------------------------------------------------- Hydra

def gpu_hydra_level(wl, wd, h_dev, root_dev, tok_dev, tree, level, rows, U_op=None, W_op=None):
    import torch

    md = _md()
    dt = md.MD_F32 if wl.dtype == "f32" else md.MD_BF16
    idx = torch.empty(rows, 1, wl.kmax, dtype=torch.int32, device="cuda")
    val = torch.empty(rows, 1, wl.kmax, dtype=torch.float32, device="cuda")
    hres = torch.empty(rows, wl.d, dtype=torch.float32, device="cuda")
    ws = torch.empty(md.md_heads_workspace_bytes(1, dt, wl.B, wl.d, wl.V, wl.K, wl.kmax), dtype=torch.uint8,
                     device="cuda")
    md.md_medusa_heads(1, dt, wl.B, wl.d, wl.V, wl.K, wl.topk, level, tree, h_dev, wd["W"], wd["b"], wd["U"], wd["E"],
                       root_dev, tok_dev, idx, val, hres, ws, U_op=U_op, W_op=W_op)
    torch.cuda.synchronize()
    return from_dev(idx), from_dev(val), from_dev(hres)


def check_hydra(wl, seed, requests=None, op=False):
    md = _md()
    topo = wl.topology()
    w = weights(wl, seed)
    x = step_inputs(wl, seed)
    ref = oracle.hydra_expand(w["W"], w["b"], w["U"], w["E"], x["h"], topo.parent, topo.rank, wl.topk,
                              x["root_tok"], x["lens"], requests=requests, want_logits=True)
    wd = {k: to_dev(v) for k, v in w.items()}
    U_op = md.operand_order(wd["U"]) if op else None
    W_op = md.operand_order(wd["W"]) if op else None
    tree = md.make_tree(topo.parent, topo.rank)
    tok_dev = to_dev(np.where(ref["tree_tok"] < 0, 0, ref["tree_tok"]).astype(np.int32))  # oracle's upstream tokens
    h_dev, root_dev = to_dev(x["h"]), to_dev(x["root_tok"])
    tau, tol = TAU[wl.dtype], TOL[wl.dtype]
    reqs = list(range(wl.B)) if requests is None else list(requests)
    for li, lvl in enumerate(ref["levels"]):
        level = li + 1
        P = len(oracle.hydra_rows(topo.parent, level))
        gi, gv, gh = gpu_hydra_level(wl, wd, h_dev, root_dev, tok_dev, tree, level, wl.B * P, U_op=U_op, W_op=W_op)
        if op:  # the residual reads W's operand-order copy in the same order as W itself: the same bits
            gi0, gv0, gh0 = gpu_hydra_level(wl, wd, h_dev, root_dev, tok_dev, tree, level, wl.B * P, U_op=U_op)
            assert np.array_equal(gi, gi0) and np.array_equal(gv.view(np.uint32), gv0.view(np.uint32))
            assert np.array_equal(gh.view(np.uint32), gh0.view(np.uint32))
        # GPU rows are (b, parent) over all requests; pick the oracle's rows
        sel = [b * P + j for b in reqs for j in range(P)]
        assert len(sel) == len(lvl["rows"])
        lg = lvl["logits"]
        ties = check_topk(gi[sel, 0], gv[sel, 0], lvl["idx"], lvl["val"], lvl["margin"], wl.topk[level - 1], tau, tol,
                          logits_of=lambda r, ii: lg[r, ii])
        err = rel_err(gh[sel], lvl["hres"])
        assert err <= tol, "level %d h' relative error %.3g" % (level, err)
        print("Hydra level %d: rows %d, h' rel err %.2e, near ties %d" % (level, len(sel), err, ties))


def test_hydra_small():
    wl = replace(HYDRA_B4, name="hydra small", B=3, d=256, V=3001, topk=(5, 3, 2, 1), N=20)
    check_hydra(wl, 31)


def test_hydra_full_size_sampled():
    # full Hydra shape (B = 4, d = 4096, V = 128,256); the oracle checks request 0's 41 rows
    check_hydra(HYDRA_B4, 41, requests=[0])


@pytest.mark.parametrize("B", [1, 3])
def test_hydra_out_of_vocabulary_parent_tokens(B):
    """A parent token outside [0, V) reads as a zero embedding: level 2 with parent tokens -1 and
    V + 5 planted among valid ones, against the oracle's residual on x = [h ; 0] for those rows.
    B = 1 runs its 3 rows on the GEMV, B = 3 its 9 rows on the matrix cores."""
    import torch

    md = _md()
    wl = replace(HYDRA_B4, name="hydra oov", B=B, d=256, V=3001, topk=(5, 3, 2, 1), N=20)
    topo = wl.topology()
    w = weights(wl, 33)
    x = step_inputs(wl, 33)
    level = 2
    parents = oracle.hydra_rows(topo.parent, level)
    P = len(parents)
    tok = synth.randint(33, 86, B * topo.n, 0, wl.V - 1).reshape(B, topo.n)  # inclusive bounds
    bad = {}
    for bi in range(B):
        for j, p in enumerate(parents):
            if (bi + j) % 3 == 0:
                tok[bi, p] = -1 if j % 2 == 0 else wl.V + 5
                bad[(bi, j)] = True
    wd = {k: to_dev(v) for k, v in w.items()}
    tree = md.make_tree(topo.parent, topo.rank)
    gi, gv, gh = gpu_hydra_level(wl, wd, to_dev(x["h"]), to_dev(x["root_tok"]), to_dev(tok), tree, level, B * P)
    hd = synth.bf16_to_f32(x["h"]).astype(np.float64)
    Ed = synth.bf16_to_f32(w["E"]).astype(np.float64)
    xs, base = [], []
    for bi in range(B):
        for j, p in enumerate(parents):
            e = np.zeros(wl.d) if (bi, j) in bad else Ed[tok[bi, p]]
            xs.append(np.concatenate([hd[bi], e]))
            base.append(hd[bi])
    ref = oracle.residual(w["W"][level - 1], w["b"][level - 1], np.array(xs), np.array(base))
    err = rel_err(gh, ref)
    assert err <= TOL[wl.dtype], "h' relative error %.3g" % err
    assert bad and len(bad) < B * P
    torch.cuda.synchronize()


def test_hydra_small_operand_order():
    # batch 3: levels of 3, 9, 15 and 15 rows, all on the matrix cores with the operand-order copy
    wl = replace(HYDRA_B4, name="hydra small", B=3, d=256, V=3001, topk=(5, 3, 2, 1), N=20)
    check_hydra(wl, 32, op=True)


def test_hydra_full_size_sampled_operand_order():
    # the full Hydra shape reading the operand-order copy of U (4 / 32 / 56 / 72 rows per level)
    check_hydra(HYDRA_B4, 42, requests=[1], op=True)


# ------------------------------------------------- many rows: matrix cores

MFMA_BF16 = Workload("mfma bf16: d=256 V=1000 K=3", "medusa", B=1, d=256, V=1000, K=3, dtype="bf16",
                     topk=(6, 3, 1), N=10, Hq=4, Hkv=1, hd=64, L=10)


@pytest.mark.parametrize("wl,M", [(MFMA_BF16, 8), (MFMA_BF16, 130),
                                  (replace(MFMA_BF16, d=512, V=5003, topk=(16, 2, 9)), 37),
                                  (replace(MFMA_BF16, d=128, V=140001, K=2, topk=(10, 3)), 9),
                                  (replace(MFMA_BF16, V=20011, K=1, topk=(10,)), 250),
                                  (replace(MFMA_BF16, d=512, V=5003, topk=(16, 2, 9)), 65),
                                  (replace(MFMA_BF16, V=4099, topk=(10, 4, 1)), 72),
                                  (replace(MFMA_BF16, d=512, V=3001, topk=(12, 5, 2)), 80),
                                  (replace(MFMA_BF16, V=4099, topk=(10, 4, 1)), 81),
                                  (replace(MFMA_BF16, d=256, V=3001, topk=(5, 2, 1)), 88),
                                  (replace(MFMA_BF16, d=128, V=3001, topk=(5, 2, 1)), 100),
                                  (replace(MFMA_BF16, V=2053, K=1, topk=(7,)), 128)])
def test_heads_medusa_mfma_rows(wl, M):
    """Eight or more bf16 rows run the MFMA path (ragged row and vocabulary tiles; V = 140,001
    leaves more than 1,024 partial lists per row for the merge). 250 rows of one head over 79
    vocabulary tiles would run every tile of a row before any bound exists, so they take the
    two-product narrow kernel (four row tiles) instead of the certified pass. 65 to 128 rows run
    the register-streamed kernel with all rows in one tile (5 to 8 column blocks; 65 and 81 leave
    one valid column in the last block, 80 fills five; at d = 128, 100 rows fill exactly one
    prefetch ring of 4 K steps; at d = 256, 72, 81 and 88 rows end their ring of 6 steps with a
    tail of 2)."""
    seed = 2000 + M
    w = weights(wl, seed)
    h = synth.normal(seed, 78, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi, gv, gh, ref, label="%s M=%d" % (wl.name, M))
    gi2, gv2, gh2 = gpu_heads_medusa(wl, wd, to_dev(h), M)
    assert np.array_equal(gi, gi2) and np.array_equal(gv.view(np.uint32), gv2.view(np.uint32))
    # with the tile norms of U the certified pass (130 rows) skips its own norms; the lists come
    # from the same exact re-scoring, so they are the same bit for bit (other paths ignore them)
    gi3, gv3, _ = gpu_heads_medusa(wl, wd, to_dev(h), M, U_norms=_md().vocab_tile_norms(wd["U"]))
    assert np.array_equal(gi, gi3) and np.array_equal(gv.view(np.uint32), gv3.view(np.uint32))


@pytest.mark.parametrize("wl_name,M,rows", [("8b", 64, [0, 31, 63]),
                                             # 40 rows of d = 8,192: the residual staged in LDS (8 chunks)
                                             ("70b", 40, [0, 17, 39]),
                                             ("70b", 512, list(range(192, 256)) + [0, 130, 300, 511])])
def test_heads_medusa_mfma_full_size_sampled(wl_name, M, rows):
    """The 70B-shaped heads over all 512 tree nodes of a batch of 8 on the certified pass: every row
    of one request (the 64 nodes of request 3) and one row in each 128-row tile checked against the
    oracle (lists, values and h')."""
    wl = LLAMA8B if wl_name == "8b" else LLAMA70B
    w = weights(wl, 8 if wl_name == "8b" else 70)
    h = synth.normal(91, 79, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, rows=rows, want_logits=True)
    ref["hres"] = ref["hres"]
    compare_medusa(wl, gi[rows], gv[rows], gh[:, rows], ref, label="%s M=%d rows %s" % (wl.name, M, rows))
    # the certified pass reading the tile norms: every list and value of all M rows the same; the
    # residual reading the operand-order copy of W: the same bits (h' too)
    md = _md()
    gi2, gv2, gh2 = gpu_heads_medusa(wl, wd, to_dev(h), M, U_norms=md.vocab_tile_norms(wd["U"]),
                                     W_op=md.operand_order(wd["W"]))
    assert np.array_equal(gi, gi2) and np.array_equal(gv.view(np.uint32), gv2.view(np.uint32))
    assert np.array_equal(gh.view(np.uint32), gh2.view(np.uint32))
    del wd


def test_heads_certified_pass_wide_contraction():
    """512 rows x 2 heads at d = 16,384, twice the 70B width, on the certified single-product pass:
    its rounding allowance grows with the contraction length, so the lists stay those of the
    float32 re-scored logits (rows of every 128-row tile checked against the oracle)."""
    md = _md()
    wl = Workload("certified d=16384 V=3001 K=2", "medusa", B=1, d=16384, V=3001, K=2, dtype="bf16",
                  topk=(10, 4), N=10, Hq=4, Hkv=1, hd=64, L=10)
    M = 512
    rows = [0, 1, 64, 127, 128, 200, 255, 256, 300, 383, 384, 450, 511]
    assert md.md_certified_rounding_allowance(wl.d) > md.md_certified_rounding_allowance(8192)
    w = weights(wl, 4400)
    h = synth.normal(4400, 86, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, rows=rows, want_logits=True)
    compare_medusa(wl, gi[rows], gv[rows], gh[:, rows], ref, label="certified d=16384 M=%d" % M)
    gi2, gv2, _ = gpu_heads_medusa(wl, wd, to_dev(h), M)
    assert np.array_equal(gi, gi2) and np.array_equal(gv.view(np.uint32), gv2.view(np.uint32))
    gi3, gv3, _ = gpu_heads_medusa(wl, wd, to_dev(h), M, U_norms=md.vocab_tile_norms(wd["U"]))
    assert np.array_equal(gi, gi3) and np.array_equal(gv.view(np.uint32), gv3.view(np.uint32))
    del wd


@pytest.mark.parametrize("nmat,V,d", [(2, 1000, 512), (1, 256, 64), (3, 513, 8192)])
def test_vocab_tile_norms(nmat, V, d):
    """md_vocab_tile_norms against float64 on the host: each 256-row tile's largest sum of squares
    (the last tile ragged at V = 1,000 and 513)."""
    md = _md()
    U = synth.normal(4500 + V, 87, (nmat, V, d), 1.0, "bf16")
    Uf = synth.bf16_to_f32(U).astype(np.float64)
    n2 = (Uf * Uf).sum(axis=2)  # [nmat, V]
    tiles = (V + 255) // 256
    ref = np.stack([[n2[m, 256 * t:256 * t + 256].max() for t in range(tiles)] for m in range(nmat)])
    got = from_dev(md.vocab_tile_norms(to_dev(U)))
    assert got.shape == (nmat, tiles)
    assert np.max(np.abs(got - ref) / ref) <= 1e-5


# ------------------------------------- operand-order copy of the projection

def test_operand_order_layout():
    """The copy's layout, bit for bit: [matrix][tile of 256 rows][step of 32 columns][16-row block]
    [lane][8] with lane l holding row l % 16 and columns 8 (l / 16) .. + 7; padded rows are zero."""
    md = _md()
    nmat, rows, cols = 2, 300, 96
    src = synth.normal(7, 5, (nmat, rows, cols), 1.0, "bf16")
    dst = from_dev(md.operand_order(to_dev(src)))
    tiles = (rows + 255) // 256
    pad = np.zeros((nmat, tiles * 256, cols), dtype=src.dtype)
    pad[:, :rows] = src
    # rows -> (tile, block, r); columns -> (step, g, e); lane = 16 g + r
    x = pad.reshape(nmat, tiles, 16, 16, cols // 32, 4, 8)
    want = x.transpose(0, 1, 4, 2, 5, 3, 6).reshape(-1)
    assert dst.dtype == src.dtype and dst.size == md.md_operand_order_bytes(nmat, rows, cols) // 2
    assert np.array_equal(dst.reshape(-1), want)


OP_CASES = [(SMALL_BF16, 1), (SMALL_BF16, 2), (SMALL_BF16, 4), (replace(SMALL_BF16, V=1111), 7), (MFMA_BF16, 8),
            (replace(MFMA_BF16, d=512, V=5003, topk=(16, 2, 9)), 37),
            (replace(MFMA_BF16, d=128, V=140001, K=2, topk=(10, 3)), 9),
            (replace(MFMA_BF16, d=512, V=5003, topk=(16, 2, 9)), 65),
            (replace(MFMA_BF16, V=4099, topk=(10, 4, 1)), 72),
            (replace(MFMA_BF16, d=128, V=3001, topk=(5, 2, 1)), 100),
            (replace(MFMA_BF16, V=2053, K=1, topk=(7,)), 128),
            (replace(MFMA_BF16, V=20011, K=1, topk=(10,)), 250),
            (replace(MFMA_BF16, V=3001, topk=(6, 3, 1), shared_u=True), 30),
            (replace(MFMA_BF16, d=512, V=5003, topk=(16, 2, 9), shared_u=True), 3),
            (replace(MFMA_BF16, V=3001, topk=(6, 3, 1), shared_u=True), 1),
            (replace(MFMA_BF16, d=512, V=5003, topk=(16, 2, 9), shared_u=True), 4)]


@pytest.mark.parametrize("wl,M", OP_CASES, ids=["%s%s M=%d" % (w.name, " shared" if w.shared_u else "", m)
                                                 for w, m in OP_CASES])
def test_heads_operand_order(wl, M):
    """The heads reading the operand-order copy of U: one row keeps the GEMV (the copy is not read),
    2 to 7 rows move from the GEMV to the matrix cores (one row through a shared projection keeps the
    GEMV residual, which then also writes the hi/lo split); from 8 rows on the same kernels run on the packed copy, so the lists and values are
    the row-major run's, bit for bit (the copy only moves where each fragment is loaded from)."""
    md = _md()
    seed = 5000 + M
    w = weights(wl, seed)
    h = synth.normal(seed, 84, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    U_op = md.operand_order(wd["U"])
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M, U_op=U_op)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi, gv, gh, ref, label="operand order %s M=%d" % (wl.name, M))
    gi2, gv2, _ = gpu_heads_medusa(wl, wd, to_dev(h), M, U_op=U_op)
    assert np.array_equal(gi, gi2) and np.array_equal(gv.view(np.uint32), gv2.view(np.uint32))
    if M >= 8:
        gi3, gv3, _ = gpu_heads_medusa(wl, wd, to_dev(h), M)
        assert np.array_equal(gi, gi3) and np.array_equal(gv.view(np.uint32), gv3.view(np.uint32))


def test_heads_many_rows_wide_residual():
    """2,000 rows x 4 heads at d = 1,024: enough whole 256 x 128 tiles that the residual runs the
    pipelined wide kernel without a split contraction (the last row tile holds 80 rows); every 7th
    row and the last are checked against the oracle, h' and lists."""
    wl = Workload("wide residual: d=1024 V=3001 K=4", "medusa", B=1, d=1024, V=3001, K=4, dtype="bf16",
                  topk=(10, 4, 2, 1), N=10, Hq=4, Hkv=1, hd=64, L=10)
    M = 2000
    rows = list(range(0, M, 7)) + [M - 1]
    w = weights(wl, 4300)
    h = synth.normal(4300, 85, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, rows=rows, want_logits=True)
    compare_medusa(wl, gi[rows], gv[rows], gh[:, rows], ref, label="wide residual M=%d" % M)


# ------------------------------------------- one projection shared by the heads

@pytest.mark.parametrize("wl,M", [(replace(TINY_F32, shared_u=True), 1), (replace(TINY_F32, shared_u=True), 3),
                                  (replace(SMALL_BF16, shared_u=True), 1), (replace(SMALL_BF16, shared_u=True), 2),
                                  (replace(MFMA_BF16, shared_u=True), 8),
                                  (replace(MFMA_BF16, d=512, V=5003, topk=(16, 2, 9), shared_u=True), 37),
                                  (replace(MFMA_BF16, V=3001, topk=(6, 3, 1), shared_u=True), 30)])
def test_heads_shared_projection(wl, M):
    """One U [V, d] for every head: the K x M vectors h' share the pass over U (GEMV rows and MFMA
    columns of several heads, each with its own top-k width; 3 heads x 30 rows = 90 columns run
    the register-streamed kernel)."""
    seed = 3000 + M
    w = weights(wl, seed)
    assert w["U"].ndim == 2
    h = synth.normal(seed, 80, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi, gv, gh, ref, label="shared %s M=%d" % (wl.name, M))


def test_heads_shared_projection_full_size():
    """The 70B-shaped heads with one 2.1 GB projection, batch 1 (the whole vocabulary checked)."""
    wl = LLAMA70B_SHARED
    w = weights(wl, 71)
    h = step_inputs(wl, 71)["h"]
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), 1)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi, gv, gh, ref, label=wl.name)
    del wd


def test_heads_shared_projection_full_size_operand_order():
    """The 70B-shaped shared projection at batch 1 with an operand-order copy of U: the GEMV
    residual, then the 4 heads' h' as 4 columns of the narrow matrix-core kernel."""
    md = _md()
    wl = LLAMA70B_SHARED
    w = weights(wl, 73)
    h = step_inputs(wl, 73)["h"]
    wd = {k: to_dev(v) for k, v in w.items()}
    U_op = md.operand_order(wd["U"])
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), 1, U_op=U_op)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi, gv, gh, ref, label=wl.name + " operand order")
    del wd, U_op


def test_heads_shared_projection_many_rows_sampled():
    """512 rows x 4 heads through one projection on the matrix cores (sampled rows)."""
    wl = LLAMA70B_SHARED
    M, rows = 512, [0, 257, 511]
    w = weights(wl, 72)
    h = synth.normal(92, 79, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, rows=rows, want_logits=True)
    compare_medusa(wl, gi[rows], gv[rows], gh[:, rows], ref, label="%s M=%d rows %s" % (wl.name, M, rows))
    gi2, gv2, _ = gpu_heads_medusa(wl, wd, to_dev(h), M, U_norms=_md().vocab_tile_norms(wd["U"]))
    assert np.array_equal(gi, gi2) and np.array_equal(gv.view(np.uint32), gv2.view(np.uint32))
    del wd


# ------------------------------------------------------------- edge cases

EIGHT = Workload("eight heads: d=256 V=3001 K=8", "medusa", B=1, d=256, V=3001, K=8, dtype="bf16",
                 topk=(16, 9, 5, 4, 3, 2, 1, 1), N=10, Hq=4, Hkv=1, hd=64, L=10)


@pytest.mark.parametrize("M", [1, 2, 16])
def test_heads_eight_heads(M):
    """The largest head count the boundary takes (K = 8), on the fused one-row launch (8 block groups),
    the GEMV (2 rows) and MFMA (16 rows) paths."""
    wl = EIGHT
    w = weights(wl, 4000 + M)
    h = synth.normal(4000 + M, 81, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi, gv, gh, ref, label="K=8 M=%d" % M)


def test_heads_many_rows_without_matrix_cores():
    """Nine bf16 rows at d = 200 (not a whole number of 128-wide tiles): the GEMV path in several passes."""
    wl = Workload("d=200 bf16", "medusa", B=1, d=200, V=2500, K=2, dtype="bf16", topk=(7, 3), N=4, Hq=4, Hkv=1,
                  hd=64, L=10)
    M = 9
    w = weights(wl, 4100)
    h = synth.normal(4100, 82, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi, gv, gh, ref, label="d=200 M=9")


@pytest.mark.parametrize("V,M,topk", [(3000, 136, (5, 3)), (10000, 520, (5, 3, 2, 1))])
def test_heads_many_rows_all_logits_tied(V, M, topk):
    """Every vocabulary row equal: every logit of a row ties, so the certified pass keeps more than 512
    survivors (V = 3000, 136 rows) or overflows its candidate buffer (V = 10000 over 520 rows and 4
    heads: 20 row tiles, so few enough vocabulary tiles per row run before the bounds exist for the
    certified pass to be chosen); both fall back to the exact scan and must return the lowest indices."""
    wl = Workload("tied vocabulary", "medusa", B=1, d=256, V=V, K=len(topk), dtype="bf16", topk=topk, N=4, Hq=4,
                  Hkv=1, hd=64, L=10)
    w = weights(wl, 4200)
    w["U"][:] = w["U"][:, :1, :]  # one row repeated
    h = synth.normal(4200, 83, (M, wl.d), 1.0, wl.dtype)
    wd = {k: to_dev(v) for k, v in w.items()}
    gi, gv, gh = gpu_heads_medusa(wl, wd, to_dev(h), M)
    ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, wl.topk, want_logits=True)
    compare_medusa(wl, gi, gv, gh, ref, label="tied V=%d" % V)
    for k, kk in enumerate(wl.topk):
        assert np.all(gi[:, k, :kk] == np.arange(kk))
