"""GPU parity of sampled decoding: the heads' full logits, the drafts drawn
from them, rejection-sampling verification and typical acceptance.

Parity rules. Floating point decides integers here in three places, each
compared with a margin from the oracle (fp64):
* a draft list whose oracle margin (the smallest gap among its k + 1 best
  perturbed values) exceeds TAU equals the oracle's list; a smaller margin
  allows only swaps of entries whose oracle values lie within TAU;
* a walk whose oracle margin (the smallest |u - acceptance probability| of
  its tests, relative |p / threshold - 1| for typical acceptance, and the gap
  of its final draw) exceeds TAU gives the oracle's accept_len, path,
  next_tok, compaction indices and cache bytes bit for bit; a smaller margin
  is counted and the outputs are checked for validity only.
The GPU works in float32 on values of order 1 (probability ratios in [0, 1],
log-probabilities and Gumbel noise below ~30), so its errors are ~1e-6 and
TAU = 1e-4 leaves two orders of magnitude. Logits: float32 sums of exact
products, compared at 1e-4 of the largest logit.
Every stage is fed the oracle's own upstream values.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from synth.topology import chain, product_order_tree
from synth.workloads import LLAMA8B, LLAMA70B, TINY_F32, step_inputs, weights

from _helpers import from_dev, to_dev

pytestmark = pytest.mark.gpu

TAU = 1e-4
LOGIT_TOL = 1e-4


def _md():
    import medusa_draft_heads_amd as md

    return md


def _words(seed, sid, *shape):
    return synth.u32(seed, sid, int(np.prod(shape))).reshape(shape)


# ------------------------------------------------------------ head logits

SMALL_BF16 = replace(LLAMA8B, name="small bf16", d=512, V=5003, B=3)
LOGIT_CASES = [("tiny f32", TINY_F32, False, None), ("bf16 3 rows ragged V", SMALL_BF16, False, None),
               ("bf16 shared projection 2 rows", replace(SMALL_BF16, B=2, shared_u=True), True, None),
               ("70B-shaped batch 1, sampled rows", LLAMA70B, False, 3000)]


@pytest.mark.parametrize("case", LOGIT_CASES, ids=[c[0] for c in LOGIT_CASES])
def test_heads_logits(case):
    import torch

    md = _md()
    name, wl, shared, sample = case
    seed = len(name)
    w = weights(wl, seed)
    h = step_inputs(wl, seed)["h"]
    kind = md.MD_HEADS_MEDUSA_SHARED if shared else md.MD_HEADS_MEDUSA
    dt = md.MD_F32 if wl.dtype == "f32" else md.MD_BF16
    M = h.shape[0]
    lg = torch.empty(M, wl.K, wl.V, dtype=torch.float32, device="cuda")
    ws = torch.empty(md.md_heads_logits_workspace_bytes(kind, M, wl.d, wl.K), dtype=torch.uint8, device="cuda")
    md.md_medusa_heads_logits(kind, dt, M, wl.d, wl.V, wl.K, to_dev(h), to_dev(w["W"]), to_dev(w["b"]),
                              to_dev(w["U"]), lg, None, ws)
    torch.cuda.synchronize()
    got = from_dev(lg)
    if sample is None:
        ref = oracle.heads_medusa(w["W"], w["b"], w["U"], h, [1] * wl.K, want_logits=True)["logits"]
    else:
        # the oracle's residual, then its projection on a sample of vocabulary rows
        rows = np.sort(np.random.default_rng(seed).choice(wl.V, sample, replace=False))
        hd = oracle.to_double(h)
        ref = np.empty((M, wl.K, rows.size))
        for k in range(wl.K):
            hres = oracle.residual(w["W"][k], w["b"][k], hd, hd)
            Uk = w["U"] if shared else w["U"][k]
            ref[:, k] = oracle.vocab_topk(np.ascontiguousarray(Uk[rows]), hres, 1, want_logits=True)[3]
        got = got[:, :, rows]
    err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    print(name, "relative error %.3g" % err)
    assert err <= LOGIT_TOL


# ------------------------------------------------------------ draft sample

def check_draft(gt, glse, ref, logits, words, kph, T):
    ties = 0
    M, K = ref["lse"].shape
    for m in range(M):
        for k in range(K):
            kk = kph[k]
            g, r = gt[m, k, :kk], ref["tok"][m, k, :kk]
            if ref["margin"][m, k] > TAU:
                assert np.array_equal(g, r), (m, k, g, r, ref["margin"][m, k])
            else:
                ties += 1
                assert len(set(g.tolist())) == kk and np.all((g >= 0) & (g < logits.shape[-1]))
                s = logits[m, k, g].astype(np.float64) / T + oracle.gumbel_from_words(words[m, k, g])
                assert np.all(np.abs(s - ref["score"][m, k, :kk]) <= TAU), (m, k)
            assert np.all(gt[m, k, kk:] == -1)
    assert np.all(np.abs(glse - ref["lse"]) <= 1e-5 * np.maximum(1.0, np.abs(ref["lse"])))
    return ties


DRAFT_CASES = [("tiny", 1, 4, 4096, (4, 2, 2, 1), 1.0, 1.0), ("70B vocab, 3 rows", 3, 4, 128256, (10, 4, 2, 1), 0.7, 1.0),
               ("lists of 16", 2, 2, 1000, (16, 3), 1.5, 1.0), ("ragged vocab", 1, 1, 140001, (16,), 1.0, 1.0),
               ("cold", 1, 2, 5000, (5, 2), 0.05, 1.0), ("peaked", 2, 3, 3001, (7, 1, 2), 1.0, 6.0),
               ("short vocab", 1, 1, 16, (16,), 1.0, 1.0)]


@pytest.mark.parametrize("case", DRAFT_CASES, ids=[c[0] for c in DRAFT_CASES])
def test_draft_sample(case):
    import torch

    md = _md()
    name, M, K, V, kph, T, scale = case
    seed = 100 + len(name)
    logits = synth.normal(seed, 31, (M, K, V), scale, "f32")
    words = _words(seed, 32, M, K, V)
    ref = oracle.draft_sample(logits, words, kph, T)
    kmax = max(kph)
    tok = torch.full((M, K, kmax), -7, dtype=torch.int32, device="cuda")
    lse = torch.empty(M, K, dtype=torch.float32, device="cuda")
    ws = torch.empty(md.md_draft_sample_workspace_bytes(M, K, V, kmax), dtype=torch.uint8, device="cuda")
    md.md_draft_sample(M, K, V, kph, T, to_dev(logits), to_dev(words), tok, lse, ws)
    torch.cuda.synchronize()
    ties = check_draft(from_dev(tok), from_dev(lse), ref, logits, words, kph, T)
    print(name, "near-tie lists", ties)


# ------------------------------------------------------------ verification

def _tree_inputs(topo, K, B, V, seed, head_scale=1.0, same=False, bad_node=None, T=1.0):
    """Target logits at every node, the drafting heads' logits, and the tree
    of tokens drawn from them (the oracle's draws)."""
    N = topo.n
    kph = [max([topo.rank[n] for n in range(N) if len(topo.paths[n]) == i] + [0]) + 1 for i in range(1, K + 1)]
    target = synth.normal(seed, 41, (B, N, V), 1.0, "f32")
    head = synth.normal(seed, 42, (B, K, V), head_scale, "f32")
    depth = [len(p) for p in topo.paths]
    if same:  # the heads' distribution is the target's at every node with children
        for n in range(N):
            if depth[n] < K:
                target[:, n] = head[:, depth[n]]
    d = oracle.draft_sample(head, _words(seed, 43, B, K, V), kph, T)
    root = synth.randint(seed, 46, B, 0, V - 1)
    tok, _ = oracle.tree_tokens_medusa(topo.parent, topo.rank, d["tok"], np.arange(B, dtype=np.int32), root,
                                       np.zeros(B, np.int32))
    if bad_node is not None:
        tok[:, bad_node] = -1
    return target, head, tok


def _run_accept_like(mode, topo, K, B, V, T, seed, dtype="bf16", Hkv=2, hd=64, L=100, head_scale=1.0, same=False,
                     eps=0.09, delta=0.3, bad_node=None):
    import torch

    md = _md()
    N = topo.n
    target, head, tok = _tree_inputs(topo, K, B, V, seed, head_scale, same, bad_node, T)
    u_words = _words(seed, 44, B, N)
    g_words = _words(seed, 45, B, V)
    if mode == "sampled":
        ref = oracle.verify_sampled(topo.parent, tok, target, head, T, u_words, g_words)
        head_lse = np.array([[oracle.logsumexp_t(head[b, k], T) for k in range(K)] for b in range(B)], np.float32)
    else:
        ref = oracle.typical_accept(topo.parent, tok, target, T, eps, delta, g_words)
    lens = np.full(B, L, np.int32)
    Lcap = L + N + 3
    acc = oracle.accept(topo.parent, K, tok, ref["chosen"], lens)
    Kc = synth.normal(seed, 2, (B, Hkv, Lcap, hd), 1.0, dtype)
    Vc = synth.normal(seed, 3, (B, Hkv, Lcap, hd), 1.0, dtype)
    rK, rV, rl = oracle.compact(Kc, Vc, lens, acc["accept_len"], acc["path"], K)
    dt = md.MD_F32 if dtype == "f32" else md.MD_BF16
    kc, vc, ld = to_dev(Kc), to_dev(Vc), to_dev(lens)
    outs = {k: torch.empty(*s, dtype=torch.int32, device="cuda") for k, s in
            (("accept_len", (B,)), ("path", (B, K + 1)), ("next_tok", (B,)), ("compact_src", (B, K + 1)))}
    tree = md.make_tree(topo.parent, topo.rank)
    if mode == "sampled":
        ws = torch.empty(md.md_verify_sampled_workspace_bytes(B, N), dtype=torch.uint8, device="cuda")
        md.md_tree_verify_sampled(tree, dt, B, K, V, Hkv, hd, Lcap, T, to_dev(target), to_dev(head), to_dev(head_lse),
                                  to_dev(tok), to_dev(u_words), to_dev(g_words), kc, vc, ld, outs["accept_len"],
                                  outs["path"], outs["next_tok"], outs["compact_src"], ws)
    else:
        ws = torch.empty(md.md_accept_typical_workspace_bytes(B, N), dtype=torch.uint8, device="cuda")
        md.md_tree_accept_typical(tree, dt, B, K, V, Hkv, hd, Lcap, T, eps, delta, to_dev(target), to_dev(tok),
                                  to_dev(g_words), kc, vc, ld, outs["accept_len"], outs["path"], outs["next_tok"],
                                  outs["compact_src"], ws)
    torch.cuda.synchronize()
    got = {k: from_dev(v) for k, v in outs.items()}
    gK, gV, gl = from_dev(kc), from_dev(vc), from_dev(ld)
    ties = 0
    for b in range(B):
        if ref["margin"][b] > TAU:
            for key in ("accept_len", "next_tok"):
                assert got[key][b] == acc[key][b], (mode, key, b, got[key][b], acc[key][b])
            for key in ("path", "compact_src"):
                assert np.array_equal(got[key][b], acc[key][b]), (mode, key, b, got[key][b], acc[key][b])
            assert np.array_equal(gK[b], rK[b]) and np.array_equal(gV[b], rV[b]) and gl[b] == rl[b]
        else:
            ties += 1
            A = got["accept_len"][b]
            assert 1 <= A <= K + 1 and 0 <= got["next_tok"][b] < V and gl[b] == L + A
            p = got["path"][b]
            assert p[0] == 0 and all(topo.parent[p[j]] == p[j - 1] for j in range(1, A)) and np.all(p[A:] == -1)
    print(mode, "accept_len", list(got["accept_len"]), "near ties", ties)
    return got, acc, ties


VERIFY_CASES = [
    ("tiny f32", "f32", ((4, 2, 2, 1), 16), 4, 6, 4096, 1.0, 1.0),
    ("64-node bf16, batch 5", "bf16", ((10, 4, 2, 1), 64), 4, 5, 3001, 1.0, 1.0),
    ("64-node, peaked heads, T 0.7", "bf16", ((10, 4, 2, 1), 64), 4, 4, 2000, 0.7, 3.0),
    ("chain", "bf16", ((1, 1, 1, 1), 5), 4, 4, 777, 1.0, 1.0),
    ("root only", "f32", ((2,), 1), 1, 3, 100, 1.0, 1.0),
    ("70B vocab, 64 nodes", "bf16", ((10, 4, 2, 1), 64), 4, 2, 128256, 1.0, 1.0),
]


@pytest.mark.parametrize("case", VERIFY_CASES, ids=[c[0] for c in VERIFY_CASES])
def test_verify_sampled(case):
    name, dtype, (kph, N), K, B, V, T, hs = case
    topo = product_order_tree(kph, N)
    _run_accept_like("sampled", topo, K, B, V, T, seed=200 + len(name), dtype=dtype, head_scale=hs)


def test_verify_sampled_draft_equal_to_target_takes_the_first_children():
    topo = product_order_tree((10, 4, 2, 1), 64)
    got, acc, ties = _run_accept_like("sampled", topo, 4, 6, 3001, 1.0, seed=7, same=True)
    assert ties == 0 and np.all(got["accept_len"] == 5)
    assert all(topo.rank[n] == 0 for b in range(6) for n in got["path"][b])


def test_verify_sampled_skips_tokens_outside_the_vocabulary():
    topo = product_order_tree((4, 2, 2, 1), 16)
    got, acc, _ = _run_accept_like("sampled", topo, 4, 4, 500, 1.0, seed=8, same=True, bad_node=1)
    assert np.all(got["path"][:, 1] == 2)  # node 1 carries -1: its sibling of rank 1 is taken instead


TYPICAL_CASES = [
    ("tiny f32", "f32", ((4, 2, 2, 1), 16), 4, 6, 4096, 1.0, 0.09, 0.3),
    ("64-node bf16, batch 5", "bf16", ((10, 4, 2, 1), 64), 4, 5, 3001, 1.0, 0.09, 0.3),
    ("64-node, T 0.5", "bf16", ((10, 4, 2, 1), 64), 4, 3, 2000, 0.5, 0.2, 0.5),
    ("chain", "bf16", ((1, 1, 1, 1), 5), 4, 4, 777, 1.0, 0.09, 0.3),
    ("70B vocab, 64 nodes", "bf16", ((10, 4, 2, 1), 64), 4, 2, 128256, 1.0, 0.09, 0.3),
]


@pytest.mark.parametrize("case", TYPICAL_CASES, ids=[c[0] for c in TYPICAL_CASES])
def test_accept_typical(case):
    name, dtype, (kph, N), K, B, V, T, eps, delta = case
    topo = product_order_tree(kph, N)
    _run_accept_like("typical", topo, K, B, V, T, seed=300 + len(name), dtype=dtype, eps=eps, delta=delta)


def test_accept_typical_limits():
    topo = product_order_tree((4, 2, 2, 1), 16)
    # threshold 0: every node matches; the deepest, lowest-index node ends the step
    got, _, _ = _run_accept_like("typical", topo, 4, 3, 1000, 1.0, seed=9, eps=0.0, delta=0.3)
    assert np.all(got["accept_len"] == 5) and np.all(got["path"][:, 4] == 12)
    # threshold 1: nothing matches
    got, _, _ = _run_accept_like("typical", topo, 4, 3, 1000, 1.0, seed=9, eps=1.0, delta=1e30)
    assert np.all(got["accept_len"] == 1)
    # a token outside the vocabulary never matches
    got, _, _ = _run_accept_like("typical", chain(4), 4, 2, 1000, 1.0, seed=10, eps=0.0, delta=0.3, bad_node=2)
    assert np.all(got["accept_len"] == 2)
