"""A whole decode step on the GPU against the oracle's whole step.

The GPU runs heads -> tree -> tree attention -> accept + compaction through
MedusaStep; the oracle runs the same step on the same inputs. The target's
verification logits are planted from the oracle's tree tokens (per-depth
acceptance a), so over several steps the GPU's accepted lengths must equal
the oracle's one for one -- and their mean estimates the closed-form E.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.workloads import (HYDRA_B4, LLAMA70B, LLAMA70B_B8, LLAMA70B_CHAIN, LLAMA70B_LMHEAD, TINY_F32, plant,
                             plant_hidden, step_inputs, weights)

from _helpers import TAU, TOL, check_topk, from_dev, rel_err, to_dev

pytestmark = pytest.mark.gpu


def make_step(wl):
    import torch

    import medusa_draft_heads_amd as md

    topo = wl.topology()
    kind = md.MD_HEADS_HYDRA if wl.kind == "hydra" else (md.MD_HEADS_MEDUSA_SHARED if wl.shared_u else md.MD_HEADS_MEDUSA)
    cfg = md.StepConfig(kind=kind,
                        dtype=torch.float32 if wl.dtype == "f32" else torch.bfloat16, B=wl.B,
                        M=wl.M if wl.kind == "medusa" else wl.B, d=wl.d, V=wl.V, K=wl.K, k_per_head=wl.topk,
                        parent=topo.parent, rank=topo.rank, Hq=wl.Hq, Hkv=wl.Hkv, hd=wl.hd, Lcap=wl.Lcap,
                        max_len=wl.L_max, target_head=wl.target_head)
    return md.MedusaStep(cfg), topo


def oracle_tree_medusa(wl, w, x, topo):
    """The oracle's heads on the rows that build the trees (with every logit)
    and its tree for this step (the tokens the logits are planted from)."""
    rows = sorted(set(int(r) for r in x["src_row"]))
    heads = oracle.heads_medusa(w["W"], w["b"], w["U"], x["h"], wl.topk, rows=rows, want_logits=True)
    full = np.full((wl.M, wl.K, wl.kmax), -1, np.int32)
    for j, r in enumerate(rows):
        full[r] = heads["idx"][j]
    tok, pos = oracle.tree_tokens_medusa(topo.parent, topo.rank, full, x["src_row"], x["root_tok"], x["lens"])
    return tok, pos, heads, rows


def medusa_check_lists(wl, heads, rows, gi, gv):
    """The GPU's lists gi [M, K, kmax] (values gv) on the rows that build the
    trees, checked against the oracle's by the margin rule. Returns the lists
    the rest of the step is checked with: the oracle's, except where a list
    within tau of a tie differs and the GPU's is valid (then the GPU's), and
    the number of such near-tie lists."""
    full = np.full((wl.M, wl.K, wl.kmax), -1, np.int32)
    ties = 0
    for j, r in enumerate(rows):
        full[r] = heads["idx"][j]
        for k in range(wl.K):
            kk = wl.topk[k]
            ties += check_topk(gi[r:r + 1, k], gv[r:r + 1, k], heads["idx"][j:j + 1, k], heads["val"][j:j + 1, k],
                               heads["margin"][j:j + 1, k], kk, TAU[wl.dtype], TOL[wl.dtype],
                               logits_of=lambda _, ii, j=j, k=k: heads["logits"][j, k, ii])
            if not np.array_equal(gi[r, k, :kk], heads["idx"][j, k, :kk]):
                full[r, k, :kk] = gi[r, k, :kk]  # a valid near-tie order: the step continues from it
    return full, ties


def hydra_levels_checked(wl, w, wd, x, xd, step, topo):
    """Hydra's levels on the GPU one call at a time (md_medusa_heads, then
    md_tree_build), each level's lists checked against the oracle's level run
    on the tree the GPU built so far (margin rule; a valid near-tie order is
    kept). Returns the tree the oracle agrees with and the near-tie count."""
    import torch

    tok = np.full((wl.B, topo.n), -1, np.int32)
    tok[:, 0] = x["root_tok"]
    depth = max(len(p) for p in topo.paths)
    ties = 0
    for level in range(1, depth + 1):
        step.heads(xd["h"], wd["W"], wd["b"], wd["U"], E=wd["E"], root_tok=xd["root_tok"], level=level,
                   U_op=wd.get("U_op"), W_op=wd.get("W_op"))
        step.build(None, xd["root_tok"], xd["lens"], level=level)
        torch.cuda.synchronize()
        lvl = oracle.hydra_level(w["W"], w["b"], w["U"], w["E"], x["h"], topo.parent, topo.rank, wl.topk, level, tok,
                                 want_logits=True)
        R = len(lvl["rows"])
        kk = wl.topk[level - 1]
        gi = from_dev(step.topk_idx)[:R, 0, :]
        gv = from_dev(step.topk_val)[:R, 0, :]
        ties += check_topk(gi, gv, lvl["idx"], lvl["val"], lvl["margin"], kk, TAU[wl.dtype], TOL[wl.dtype],
                           logits_of=lambda r, ii: lvl["logits"][r, ii])
        row_of = {rp: r for r, rp in enumerate(lvl["rows"])}
        for (b_, n) in lvl["tok"]:
            tok[b_, n] = gi[row_of[(b_, topo.parent[n])], topo.rank[n]]  # the oracle's entry, or a valid near-tie one
        gt = from_dev(step.tree_tok)
        for (b_, n) in lvl["tok"]:
            assert gt[b_, n] == tok[b_, n], (level, b_, n)
    return tok, ties


def run_and_compare(wl, w, wd, step, topo, seed, s):
    """One whole step on the GPU and the oracle's checks of every stage.
    Near-tie top-k lists (margin rule) are checked for validity and the step
    continues from the GPU's valid lists, so every later stage is still
    compared bit for bit; returns the accepted lengths."""
    import torch

    x = step_inputs(wl, seed, step=s)
    xd = {k: to_dev(v) for k, v in x.items() if k != "logits"}
    ties = 0
    if wl.kind == "hydra":
        tok, ties = hydra_levels_checked(wl, w, wd, x, xd, step, topo)
        pos = np.array([[int(x["lens"][b_]) + len(p) for p in topo.paths] for b_ in range(wl.B)], np.int32)
    else:
        tok, pos, heads, rows = oracle_tree_medusa(wl, w, x, topo)
    if wl.target_head:
        # verification through the target's LM head: plant the hidden states
        Ht = plant_hidden(x["Ht"], w["Wt"], topo, tok, wl.a, seed=seed, step=s)
        xd["Ht"] = to_dev(Ht)
        tstar, tval, tmargin = oracle.target_argmax(Ht.reshape(wl.B * topo.n, wl.d), w["Wt"])
    else:
        logits = plant(x["logits"], topo, tok, wl.a, seed=seed, step=s)
        xd["logits"] = to_dev(logits)
        tstar = oracle.argmax(logits)
    if wl.kind == "hydra":
        # the rest of the step after the levels; the whole step through MedusaStep.run is compared
        # with it below
        xd0 = {k: v.clone() for k, v in xd.items()}
        step.attention(xd["q"], xd["Kc"], xd["Vc"], xd["lens"])
        if wl.target_head:
            step.verify(xd["Ht"], wd["Wt"], wd.get("Wt_op"))
            step.accept_tokens(xd["Kc"], xd["Vc"], xd["lens"])
        else:
            step.accept(xd["logits"], xd["Kc"], xd["Vc"], xd["lens"])
    else:
        step.run(wd, xd)
    torch.cuda.synchronize()
    if wl.kind == "medusa":
        full, ties = medusa_check_lists(wl, heads, rows, from_dev(step.topk_idx), from_dev(step.topk_val))
        tok, pos = oracle.tree_tokens_medusa(topo.parent, topo.rank, full, x["src_row"], x["root_tok"], x["lens"])
    if ties:
        print("near-tie lists in this step: %d (checked valid; the step continues from the GPU's)" % ties)
    assert np.array_equal(from_dev(step.tree_tok), tok)
    assert np.array_equal(from_dev(step.tree_pos), pos)
    ref_attn = oracle.tree_attention(topo.parent, x["q"], x["Kc"], x["Vc"], x["lens"])
    ga = from_dev(step.attn_out)
    ga = ga.astype(np.float64) if wl.dtype == "f32" else synth.bf16_to_f32(ga).astype(np.float64)
    err = rel_err(ga, ref_attn)
    assert err <= TOL[wl.dtype], "attention relative error %.3g" % err
    if wl.target_head:
        # the GPU's choices must be the oracle's, or within tau of the best where the oracle's top two
        # are closer than that; acceptance is then checked on the GPU's (valid) choices
        gt = from_dev(step.target_tok).reshape(-1)
        f64 = (lambda a: synth.bf16_to_f32(a).astype(np.float64)) if wl.dtype == "bf16" else (lambda a: a.astype(np.float64))
        Hf = f64(Ht.reshape(wl.B * topo.n, wl.d))
        near = 0
        for r in range(gt.size):
            if tmargin[r] > TAU[wl.dtype]:
                assert gt[r] == tstar[r], (r, gt[r], tstar[r])
            else:
                near += 1
                assert tval[r] - float(f64(w["Wt"][gt[r]]) @ Hf[r]) <= TAU[wl.dtype]
        if near:
            print("target choices within tau of a tie: %d of %d" % (near, gt.size))
        tstar = gt.reshape(wl.B, topo.n)
    ref = oracle.accept(topo.parent, wl.K, tok, tstar, x["lens"])
    for key in ("accept_len", "path", "next_tok", "compact_src"):
        assert np.array_equal(from_dev(getattr(step, key)), ref[key]), key
    rK, rV, rl = oracle.compact(x["Kc"], x["Vc"], x["lens"], ref["accept_len"], ref["path"], wl.K)
    assert np.array_equal(from_dev(xd["Kc"]), rK) and np.array_equal(from_dev(xd["Vc"]), rV)
    assert np.array_equal(from_dev(xd["lens"]), rl)
    if wl.kind == "hydra":
        # the whole step through MedusaStep.run on fresh copies of the inputs: the same outputs, bit for bit
        outs = {k: from_dev(getattr(step, k)) for k in ("tree_tok", "attn_out", "accept_len", "path", "next_tok",
                                                        "compact_src")}
        step.run(wd, xd0)
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert np.array_equal(from_dev(getattr(step, k)), v), "MedusaStep.run differs in " + k
        assert np.array_equal(from_dev(xd0["Kc"]), rK) and np.array_equal(from_dev(xd0["lens"]), rl)
    return ref["accept_len"]


def test_step_tiny_many_steps():
    wl = TINY_F32
    seed = 3
    w = weights(wl, seed)
    wd = {k: to_dev(v) for k, v in w.items()}
    step, topo = make_step(wl)
    lens = [int(run_and_compare(wl, w, wd, step, topo, seed, s)[0]) for s in range(24)]
    print("tiny accepted lengths:", lens, "mean", np.mean(lens))


def test_step_tiny_shared_projection():
    from dataclasses import replace

    wl = replace(TINY_F32, shared_u=True)
    seed = 4
    w = weights(wl, seed)
    wd = {k: to_dev(v) for k, v in w.items()}
    step, topo = make_step(wl)
    lens = [int(run_and_compare(wl, w, wd, step, topo, seed, s)[0]) for s in range(6)]
    print("tiny shared-projection accepted lengths:", lens)


def test_step_tiny_target_head():
    from dataclasses import replace

    wl = replace(TINY_F32, target_head=True)
    seed = 5
    w = weights(wl, seed)
    wd = {k: to_dev(v) for k, v in w.items()}
    step, topo = make_step(wl)
    lens = [int(run_and_compare(wl, w, wd, step, topo, seed, s)[0]) for s in range(6)]
    print("tiny, verified through the LM head: accepted lengths", lens)


def test_step_70b_lm_head():
    wl = LLAMA70B_LMHEAD
    seed = 73
    w = weights(wl, seed)
    wd = {k: to_dev(v) for k, v in w.items()}
    step, topo = make_step(wl)
    acc = run_and_compare(wl, w, wd, step, topo, seed, 0)
    print("70B-shaped step verified through the LM head accepted", acc)


def test_step_70b_shaped():
    """Three chained 70B-shaped steps at batch 1 (the bench's workload), then the top-1 chain."""
    wl = LLAMA70B
    seed = 70
    w = weights(wl, seed)
    wd = {k: to_dev(v) for k, v in w.items()}
    step, topo = make_step(wl)
    accs = [int(run_and_compare(wl, w, wd, step, topo, seed, s)[0]) for s in range(3)]
    print("70B-shaped steps accepted", accs)
    # the top-1 chain runs on the same weights
    wlc = LLAMA70B_CHAIN
    stepc, topoc = make_step(wlc)
    acc = run_and_compare(wlc, w, wd, stepc, topoc, seed, 1)
    print("70B-shaped chain accepted", acc)


def test_step_70b_batch8():
    """The batch-8 step at full shape: heads over all 512 tree nodes (the certified matrix-core
    pass), each request's tree from its source row, attention over ragged caches (lengths drawn in
    [1,024, 4,096]), acceptance and compaction of all 8 requests, against the oracle."""
    wl = LLAMA70B_B8
    seed = 78
    w = weights(wl, seed)
    wd = {k: to_dev(v) for k, v in w.items()}
    step, topo = make_step(wl)
    acc = run_and_compare(wl, w, wd, step, topo, seed, 0)
    print("70B-shaped batch-8 step accepted", acc.tolist())
    del wd


def test_step_hydra_batch4():
    """Hydra's batch-4 step at full shape (d = 4,096, V = 128,256, 4 sequentially dependent levels
    on the operand-order copy of U, tree attention over L = 8,192), level by level against the
    oracle run on the tree the GPU built, then the whole step through MedusaStep.run."""
    import medusa_draft_heads_amd as md

    wl = HYDRA_B4
    seed = 44
    w = weights(wl, seed)
    wd = {k: to_dev(v) for k, v in w.items()}
    wd["U_op"] = md.operand_order(wd["U"])
    wd["W_op"] = md.operand_order(wd["W"])
    step, topo = make_step(wl)
    acc = run_and_compare(wl, w, wd, step, topo, seed, 0)
    print("Hydra batch-4 step accepted", acc.tolist())
    del wd


def test_step_hydra_small():
    from dataclasses import replace

    wl = replace(HYDRA_B4, name="hydra small", B=2, d=256, V=2048, N=20, L=300)
    seed = 12
    w = weights(wl, seed)
    wd = {k: to_dev(v) for k, v in w.items()}
    step, topo = make_step(wl)
    for s in range(3):
        run_and_compare(wl, w, wd, step, topo, seed, s)


@pytest.mark.parametrize("wlname", ["tiny_sampled", "tiny_typical"])
def test_sampled_step_tiny(wlname):
    """A whole sampled step (heads' logits -> drafts drawn -> tree -> attention
    -> rejection-sampling walk or typical acceptance -> compaction) against the
    oracle's, over three steps. Each stage of the oracle is fed its own
    upstream values; near ties (margin rule) are counted and checked valid."""
    import torch

    import medusa_draft_heads_amd as md
    from synth.workloads import ALL

    wl = ALL[wlname]
    topo = wl.topology()
    cfg = md.StepConfig(kind=md.MD_HEADS_MEDUSA, dtype=torch.float32, B=wl.B, M=wl.M, d=wl.d, V=wl.V, K=wl.K,
                        k_per_head=wl.topk, parent=topo.parent, rank=topo.rank, Hq=wl.Hq, Hkv=wl.Hkv, hd=wl.hd,
                        Lcap=wl.Lcap, max_len=wl.L_max, verify=wl.verify, temperature=wl.temperature, eps=wl.eps,
                        delta=wl.delta)
    step = md.MedusaStep(cfg)
    seed = 12
    w = weights(wl, seed)
    wd = {k: to_dev(v) for k, v in w.items()}
    lens_seen = []
    for s in range(3):
        x = step_inputs(wl, seed, step=s)
        if wl.verify == "sampled":
            heads = oracle.heads_medusa(w["W"], w["b"], w["U"], x["h"], [1] * wl.K, want_logits=True)
            dr = oracle.draft_sample(heads["logits"], x["draft_words"], wl.topk, wl.temperature)
            full = dr["tok"]
        else:
            heads = oracle.heads_medusa(w["W"], w["b"], w["U"], x["h"], wl.topk)
            full = heads["idx"]
        tok, pos = oracle.tree_tokens_medusa(topo.parent, topo.rank, full, x["src_row"], x["root_tok"], x["lens"])
        xd = {k: to_dev(v) for k, v in x.items()}
        step.run(wd, xd)
        torch.cuda.synchronize()
        if wl.verify == "sampled":
            assert float(np.max(np.abs(from_dev(step.head_logits) - heads["logits"]))) <= 1e-5 * float(
                np.max(np.abs(heads["logits"])))
            assert np.min(dr["margin"]) > TAU["f32"] or pytest.skip("near-tie draft list")
            ref = oracle.verify_sampled(topo.parent, tok, x["logits"], heads["logits"], wl.temperature, x["u_words"],
                                        x["g_words"])
        else:
            assert np.min(heads["margin"]) > TAU["f32"] or pytest.skip("near-tie top-k list")
            ref = oracle.typical_accept(topo.parent, tok, x["logits"], wl.temperature, wl.eps, wl.delta,
                                        x["g_words"])
        assert np.array_equal(from_dev(step.tree_tok), tok)
        acc = oracle.accept(topo.parent, wl.K, tok, ref["chosen"], x["lens"])
        if ref["margin"][0] > 1e-4:
            for key in ("accept_len", "path", "next_tok", "compact_src"):
                assert np.array_equal(from_dev(getattr(step, key)), acc[key]), key
            rK, rV, rl = oracle.compact(x["Kc"], x["Vc"], x["lens"], acc["accept_len"], acc["path"], wl.K)
            assert np.array_equal(from_dev(xd["Kc"]), rK) and np.array_equal(from_dev(xd["lens"]), rl)
        lens_seen.append(int(from_dev(step.accept_len)[0]))
    print(wlname, "accept_len per step", lens_seen)
