"""Pins of the CPU oracle to what the pages and mathematics fix.

Each test checks the oracle against something other than itself: numbers the
pages print (tests/golden, each with its citation), closed forms and textbook
values, library routines that compute a special case, invariants, and the
tree-attention identity (every root-to-leaf path run as its own causal
sequence gives the same outputs).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.topology import chain, product_order_tree
from synth.workloads import plant, plant_hidden

from conftest import GOLDEN


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------ byte accounting

def test_head_parameter_counts_match_page():
    g = golden("head_params.json")
    d, V, K = g["d"], g["V"], g["heads"]
    residual = oracle.head_weight_elems(d, d, 0)
    per_head = oracle.head_weight_elems(d, d, V)
    vocab = per_head - residual
    assert round(residual / 1e6, 1) == g["residual_params_M"]
    assert round(vocab / 1e6, 1) == g["vocab_params_M"]
    assert round(per_head / 1e6, 1) == g["per_head_params_M"]
    assert round(K * per_head / 1e9, 2) == g["total_params_B"]
    assert round(K * per_head * 2 / 1e9, 2) == g["total_bytes_GB_bf16"]
    assert round(100 * K * per_head * 2 / (g["target_bytes_GB"] * 1e9), 1) == g["heads_share_of_step_pct"]
    assert round(100 * vocab / per_head) == g["vocab_share_of_head_params_pct"]
    assert round((K - 1) * vocab / 1e9, 2) == g["shared_projection_saving_B"]
    # the exact integers behind the printed figures
    assert (residual, vocab, per_head, K * per_head) == (67_117_056, 1_050_673_152, 1_117_790_208, 4_471_160_832)


def test_ridge_arithmetic_matches_page():
    g = golden("ridge.json")
    ridge = g["h100_dense_bf16_tflops"] * 1e12 / (g["h100_hbm_tb_s"] * 1e12)
    assert abs(ridge - g["ridge_tokens_approx"]) < 1.0
    assert g["tree_nodes"] * g["batch"] == g["tree_tokens_at_batch"] > ridge
    assert abs(ridge / g["draft_chain_tokens"] - g["draft_chain_free_batch_approx"]) < 1.0


# ------------------------------------------------------------ residual block

def _rand_bf16(seed, shape, std):
    return synth.normal(seed, 1, shape, std, "bf16")


def test_residual_zero_weights_is_identity():
    d = 64
    h = synth.normal(1, 1, (3, d), 1.0, "f32")
    W = np.zeros((d, d), np.float32)
    b = np.zeros(d, np.float32)
    hd = h.astype(np.float64)
    assert np.array_equal(oracle.residual(W, b, hd, hd), hd)


def test_residual_silu_textbook_values():
    # W = 0 and a constant bias c leave hres = h + SiLU(c); SiLU(1) = 1/(1+e^-1),
    # SiLU(-2) = -2/(1+e^2) (textbook logistic values)
    d = 8
    h = np.linspace(-1, 1, d, dtype=np.float32)[None, :]
    hd = h.astype(np.float64)
    W = np.zeros((d, d), np.float32)
    for c, want in ((1.0, 0.7310585786300049), (-2.0, -0.2384058440442351), (0.0, 0.0)):
        b = np.full(d, c, np.float32)
        got = oracle.residual(W, b, hd, hd) - hd
        assert np.allclose(got, want, rtol=0, atol=1e-15)
    # a very negative bias switches the block off
    b = np.full(d, -40.0, np.float32)
    assert np.max(np.abs(oracle.residual(W, b, hd, hd) - hd)) < 1e-15


def test_residual_silu_odd_part():
    # SiLU(x) - SiLU(-x) = x, so with W = I, b = 0: hres(h) - hres(-h) = 3h
    d = 32
    h = synth.normal(2, 1, (2, d), 1.0, "f32").astype(np.float64)
    W = np.eye(d, dtype=np.float32)
    b = np.zeros(d, np.float32)
    diff = oracle.residual(W, b, h, h) - oracle.residual(W, b, -h, -h)
    assert np.allclose(diff, 3 * h, rtol=0, atol=1e-13)


def test_residual_orientation_rows_are_outputs():
    # W[r][c] is output r, input c (the torch Linear convention)
    d = 16
    x = np.arange(d, dtype=np.float64)[None, :] + 1
    W = np.zeros((d, d), np.float32)
    W[3, 11] = 1.0
    b = np.zeros(d, np.float32)
    z = oracle.residual(W, b, x, np.zeros_like(x))
    silu = lambda t: t / (1 + math.exp(-t))
    assert abs(z[0, 3] - silu(12.0)) < 1e-12
    assert np.all(z[0, np.arange(d) != 3] == 0)


def test_residual_matches_library_matmul_bf16():
    d, din, M = 96, 192, 5
    W = _rand_bf16(5, (d, din), 1 / math.sqrt(d))
    b = _rand_bf16(6, (d,), 1 / math.sqrt(d))
    x = synth.bf16_to_f32(_rand_bf16(7, (M, din), 1.0)).astype(np.float64)
    base = x[:, :d].copy()
    Wf = synth.bf16_to_f32(W).astype(np.float64)
    bf = synth.bf16_to_f32(b).astype(np.float64)
    z = x @ Wf.T + bf
    ref = base + z / (1 + np.exp(-z))
    got = oracle.residual(W, b, x, base)
    assert np.max(np.abs(got - ref)) < 1e-12


# ------------------------------------------------------------- top-k lists

def test_topk_identity_projection_is_argsort():
    d = 200
    h = synth.normal(8, 1, (2, d), 1.0, "f32").astype(np.float64)
    U = np.eye(d, dtype=np.float32)
    idx, val, margin, _ = oracle.vocab_topk(U, h, 10)
    for m in range(2):
        ref = np.argsort(-h[m], kind="stable")[:10]
        assert np.array_equal(idx[m], ref)
        assert np.array_equal(val[m], h[m][ref])
        s = np.sort(h[m])[::-1][:11]
        assert margin[m] == np.min(s[:-1] - s[1:])


def test_topk_ties_break_to_lower_index():
    # duplicated projection rows give exactly equal logits
    d, V = 8, 40
    rng = np.random.default_rng(1)
    base = rng.integers(-3, 4, size=(10, d)).astype(np.float32)
    U = base[rng.integers(0, 10, size=V)]
    h = rng.integers(-2, 3, size=(1, d)).astype(np.float64)
    idx, val, margin, logits = oracle.vocab_topk(U, h, 16, want_logits=True)
    ref = np.lexsort((np.arange(V), -logits[0]))[:16]
    assert np.array_equal(idx[0], ref)
    assert margin[0] == 0.0


def test_topk_matches_library_sort_bf16():
    d, V = 128, 3000
    U = _rand_bf16(9, (V, d), 1 / math.sqrt(d))
    h = synth.normal(10, 1, (3, d), 1.0, "f32").astype(np.float64)
    idx, val, margin, _ = oracle.vocab_topk(U, h, 12)
    logits = h @ synth.bf16_to_f32(U).astype(np.float64).T
    for m in range(3):
        assert margin[m] > 1e-9
        ref = np.argsort(-logits[m], kind="stable")[:12]
        assert np.array_equal(idx[m], ref)
        assert np.allclose(val[m], logits[m][ref], rtol=0, atol=1e-12)


def test_shared_projection_with_zero_residual_is_one_library_sort():
    # one U for every head ("What interviewers probe next"); with W = 0 and
    # b = 0 every head's h' is h, so head k's list is the first k_k entries of
    # a single library sort of U h, and h' equals h exactly
    d, V, K = 64, 2000, 3
    topk = (7, 3, 1)
    W = np.zeros((K, d, d), np.uint16)
    b = np.zeros((K, d), np.uint16)
    U = _rand_bf16(21, (V, d), 1 / math.sqrt(d))
    h = _rand_bf16(22, (4, d), 1.0)
    out = oracle.heads_medusa(W, b, U, h, topk)
    hf = synth.bf16_to_f32(h).astype(np.float64)
    logits = hf @ synth.bf16_to_f32(U).astype(np.float64).T
    for k in range(K):
        assert np.array_equal(out["hres"][k], hf)
        for m in range(4):
            ref = np.argsort(-logits[m], kind="stable")[: topk[k]]
            assert np.array_equal(out["idx"][m, k, : topk[k]], ref)
            assert np.all(out["idx"][m, k, topk[k]:] == -1)


def test_target_argmax_identity_head_is_library_argmax():
    # an identity LM head (V = d) makes the logits the hidden state itself: the
    # choice is the library's first-index argmax, ties included
    d = 64
    H = synth.normal(23, 1, (5, d), 1.0, "f32")
    H[1, 10] = H[1, 40] = np.float32(9.0)  # an exact tie: the lower index wins
    tok, val, margin = oracle.target_argmax(H, np.eye(d, dtype=np.float32))
    assert np.array_equal(tok, np.argmax(H, axis=1))
    assert tok[1] == 10 and margin[1] == 0.0
    assert np.array_equal(val, H.max(axis=1).astype(np.float64))


def test_hydra_level1_with_zero_embedding_half_is_medusa():
    # Hydra's input is [h ; E[token]]; with the E half of W zeroed, level 1
    # computes exactly a Medusa head with the h half of W
    d, V, K = 32, 500, 2
    topk = (4, 2)
    topo = product_order_tree(topk, 7)
    W = _rand_bf16(11, (K, d, 2 * d), 1 / math.sqrt(d))
    W[:, :, d:] = 0
    b = _rand_bf16(12, (K, d), 1 / math.sqrt(d))
    U = _rand_bf16(13, (K, V, d), 1 / math.sqrt(d))
    E = _rand_bf16(14, (V, d), 1 / math.sqrt(d))
    h = _rand_bf16(15, (2, d), 1.0)
    root = np.array([3, 17], np.int32)
    hy = oracle.hydra_expand(W, b, U, E, h, topo.parent, topo.rank, topk, root, np.array([5, 9], np.int32))
    Wm = np.ascontiguousarray(W[:, :, :d])
    me = oracle.heads_medusa(Wm, b, U, h, topk)
    lvl1 = hy["levels"][0]
    assert [r for r in lvl1["rows"]] == [(0, 0), (1, 0)]
    assert np.array_equal(lvl1["idx"], me["idx"][:, 0, :4])
    assert np.allclose(lvl1["hres"], me["hres"][0], rtol=0, atol=1e-13)
    # depth-1 tree tokens are the root rows' lists at each node's rank
    for b_ in range(2):
        for n in range(topo.n):
            if len(topo.paths[n]) == 1:
                assert hy["tree_tok"][b_, n] == me["idx"][b_, 0, topo.rank[n]]


def _hydra_planted(V, K, seed):
    # V = d; the h half of every W is zero and its E half a permutation matrix
    # Q_i, b_i = c_i (a positive constant per head), h = 0, and head i's
    # projection is a permutation matrix P_i. Level i then gives the parent's
    # row hres[r] = SiLU(E[t][sigma_i(r)] + c_i), t the parent's token, and
    # the logits logit[v] = hres[pi_i(v)]. E rows hold a permutation of 1..V
    # scaled by 1/V (exact in bf16, all positive, distinct), and SiLU
    # increases on the positives, so head i's list for a parent with token t
    # is exactly the library's stable argsort of -E[t][sigma_i][pi_i].
    d = V
    rng = np.random.default_rng(seed)
    bf = lambda x: (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    E = np.stack([rng.permutation(V) + 1 for _ in range(V)]).astype(np.float32) / V
    sig = [rng.permutation(d) for _ in range(K)]
    pis = [rng.permutation(V) for _ in range(K)]
    c = [0.25 * (i + 1) for i in range(K)]
    W = np.zeros((K, d, 2 * d), np.float32)
    U = np.zeros((K, V, d), np.float32)
    b = np.zeros((K, d), np.float32)
    for i in range(K):
        W[i, np.arange(d), d + sig[i]] = 1.0
        U[i, np.arange(V), pis[i]] = 1.0
        b[i] = c[i]
    perm = [sig[i][pis[i]] for i in range(K)]  # logit[v] = SiLU(E[t][perm_i[v]] + c_i)
    return bf(W), bf(b), bf(U), bf(E), E, sig, perm, c


def test_hydra_rows_parent_sets():
    # a hand-built topology: root; two depth-1 nodes, the first with two
    # children and the second with one; one depth-3 node under node 3
    parent = [-1, 0, 0, 1, 1, 2, 3]
    assert oracle.hydra_rows(parent, 1) == [0]
    assert oracle.hydra_rows(parent, 2) == [1, 2]
    assert oracle.hydra_rows(parent, 3) == [3]
    assert oracle.hydra_rows(parent, 4) == []
    # the 64-node product-order tree over (10, 4, 2, 1): parents with children
    # per level, hence rows per request for Hydra's four levels
    topo = product_order_tree((10, 4, 2, 1), 64)
    assert [len(oracle.hydra_rows(topo.parent, i)) for i in (1, 2, 3, 4)] == [1, 8, 14, 18]


@pytest.mark.parametrize("topk,n_nodes", [((4, 2, 2, 1), 16), ((10, 4, 2, 1), 64), ((3, 3, 3), 20)])
def test_hydra_levels_follow_each_nodes_own_parent_token(topk, n_nodes):
    # Hydra's heads are sequentially dependent (Hydra abstract): a node at depth
    # i takes its entry from the list head i computes for the node's own parent
    # token. With the planted weights above the expected tree is a recursion of
    # library sorts from the root token, independent of the oracle's arithmetic.
    V, K = 64, len(topk)
    W, b, U, E_bf, E, sig, perm, c = _hydra_planted(V, K, 7 + n_nodes)
    topo = product_order_tree(topk, n_nodes)
    h = np.zeros((3, V), np.uint16)
    root = np.array([5, 40, 63], np.int32)
    lens = np.array([0, 17, 1000], np.int32)
    hy = oracle.hydra_expand(W, b, U, E_bf, h, topo.parent, topo.rank, topk, root, lens)
    for r in range(3):
        want = [int(root[r])]
        for n in range(1, topo.n):
            i = len(topo.paths[n])
            parent_tok = want[topo.parent[n]]
            order = np.argsort(-E[parent_tok][perm[i - 1]], kind="stable")
            want.append(int(order[topo.rank[n]]))
        assert hy["tree_tok"][r].tolist() == want
        assert hy["tree_pos"][r].tolist() == [int(lens[r]) + len(p) for p in topo.paths]
    # every level's rows are (request, parent with children at that depth), and
    # each row's whole list is that parent's sort
    for i, lvl in enumerate(hy["levels"], start=1):
        parents = oracle.hydra_rows(topo.parent, i)
        assert lvl["rows"] == [(r, p) for r in range(3) for p in parents]
        for j, (r, p) in enumerate(lvl["rows"]):
            t = int(hy["tree_tok"][r, p])
            order = np.argsort(-E[t][perm[i - 1]], kind="stable")[: topk[i - 1]]
            assert lvl["idx"][j].tolist() == order.tolist()
            # the row itself: torch's SiLU of the gathered, shifted E row
            z = torch.from_numpy(E[t][sig[i - 1]].astype(np.float64) + c[i - 1])
            assert np.allclose(lvl["hres"][j], torch.nn.functional.silu(z).numpy(), rtol=0, atol=1e-14)


def test_hydra_parent_token_outside_vocabulary_embeds_as_zero():
    # a parent token outside [0, V) names no row of E: with h = 0 the row's
    # pre-activation is then the constant bias c_1, every logit is SiLU(c_1)
    # and the list is 0, 1, 2, ... (equal values, lower index first)
    V, K = 64, 2
    W, b, U, E_bf, _, _, _, c = _hydra_planted(V, K, 3)
    topo = product_order_tree((4, 2), 7)
    h = np.zeros((2, V), np.uint16)
    hy = oracle.hydra_expand(W, b, U, E_bf, h, topo.parent, topo.rank, (4, 2),
                             np.array([-1, V + 5], np.int32), np.array([0, 0], np.int32))
    lvl1 = hy["levels"][0]
    assert lvl1["idx"].tolist() == [[0, 1, 2, 3], [0, 1, 2, 3]]
    want = torch.nn.functional.silu(torch.tensor(c[0], dtype=torch.float64)).item()
    assert np.allclose(lvl1["hres"], want, rtol=0, atol=1e-15)


# ------------------------------------------------------------------ the tree

def test_tree_tokens_by_brute_force():
    topo = product_order_tree((4, 2, 2, 1), 16)
    M, K, kmax = 3, 4, 4
    rng = np.random.default_rng(2)
    lists = rng.integers(0, 1000, size=(M, K, kmax)).astype(np.int32)
    src_row = np.array([2, 0], np.int32)
    root = np.array([7, 8], np.int32)
    lens = np.array([100, 0], np.int32)
    tok, pos = oracle.tree_tokens_medusa(topo.parent, topo.rank, lists, src_row, root, lens)
    for b in range(2):
        for n, p in enumerate(topo.paths):
            want = root[b] if not p else lists[src_row[b], len(p) - 1, p[-1]]
            assert tok[b, n] == want and pos[b, n] == lens[b] + len(p)


# ------------------------------------------------------------ tree attention

def _path_of(parent, n):
    out = []
    while n >= 0:
        out.append(n)
        n = parent[n]
    return out[::-1]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tree_attention_equals_per_path_causal_attention(dtype):
    topo = product_order_tree((4, 2, 2, 1), 16)
    B, N, Hq, Hkv, hd = 2, 16, 4, 2, 16
    lens = np.array([6, 0], np.int32)
    Lcap = 6 + N + 3
    q = synth.normal(20, 1, (B, N, Hq, hd), 1.0, dtype)
    Kc = synth.normal(21, 1, (B, Hkv, Lcap, hd), 1.0, dtype)
    Vc = synth.normal(22, 1, (B, Hkv, Lcap, hd), 1.0, dtype)
    out = oracle.tree_attention(topo.parent, q, Kc, Vc, lens)
    f = (lambda a: a.astype(np.float64)) if dtype == "f32" else (lambda a: synth.bf16_to_f32(a).astype(np.float64))
    qd, Kd, Vd = torch.from_numpy(f(q)), torch.from_numpy(f(Kc)), torch.from_numpy(f(Vc))
    leaves = [n for n in range(N) if n not in topo.parent]
    for b in range(B):
        L = int(lens[b])
        for leaf in leaves:
            path = _path_of(topo.parent, leaf)
            slots = list(range(L)) + [L + j for j in path]
            keys = Kd[b][:, slots].repeat_interleave(Hq // Hkv, dim=0)  # [Hq, T, hd]
            vals = Vd[b][:, slots].repeat_interleave(Hq // Hkv, dim=0)
            qs = qd[b, path].permute(1, 0, 2)  # [Hq, P, hd]
            P, T = len(path), len(slots)
            mask = torch.arange(T)[None, :] < (L + 1 + torch.arange(P))[:, None]  # causal with offset L
            ref = torch.nn.functional.scaled_dot_product_attention(qs, keys, vals, attn_mask=mask)
            got = torch.from_numpy(out[b, path]).permute(1, 0, 2)
            assert torch.max(torch.abs(ref - got)).item() < 1e-12


def test_tree_attention_special_cases():
    # root only and an empty cache: the single visible key gives out = v
    q = synth.normal(30, 1, (1, 1, 2, 8), 1.0, "f32")
    Kc = synth.normal(31, 1, (1, 1, 3, 8), 1.0, "f32")
    Vc = synth.normal(32, 1, (1, 1, 3, 8), 1.0, "f32")
    out = oracle.tree_attention([-1], q, Kc, Vc, np.array([0], np.int32))
    assert np.array_equal(out[0, 0, 0], Vc[0, 0, 0].astype(np.float64))
    assert np.array_equal(out[0, 0, 1], Vc[0, 0, 0].astype(np.float64))
    # identical keys: uniform weights, so the mean of the visible values
    topo = chain(3)
    L = 5
    Kc = np.tile(synth.normal(33, 1, (1, 1, 1, 8), 1.0, "f32"), (1, 1, L + 4, 1))
    Vc = synth.normal(34, 1, (1, 1, L + 4, 8), 1.0, "f32")
    q = synth.normal(35, 1, (1, 4, 1, 8), 1.0, "f32")
    out = oracle.tree_attention(topo.parent, q, Kc, Vc, np.array([L], np.int32))
    for n in range(4):
        want = Vc[0, 0, : L + n + 1].astype(np.float64).mean(axis=0)
        assert np.allclose(out[0, n, 0], want, rtol=0, atol=1e-14)


# -------------------------------------------------------- accept / compaction

def test_argmax_first_index_on_ties():
    x = np.array([[1, 5, 5, 2], [0, 0, 0, 0], [-1, -3, -1, -2]], np.float32)
    assert list(oracle.argmax(x)) == [1, 0, 0]


def test_accept_all_and_none():
    K = 4
    topo = chain(K)
    tok = np.array([[9, 1, 2, 3, 4]], np.int32)
    lens = np.array([10], np.int32)
    # the target agrees with every draft: the chain is accepted in full
    ts = np.array([[1, 2, 3, 4, 77]], np.int32)
    r = oracle.accept(topo.parent, K, tok, ts, lens)
    assert r["accept_len"][0] == K + 1 and list(r["path"][0]) == [0, 1, 2, 3, 4]
    assert r["next_tok"][0] == 77 and list(r["compact_src"][0]) == [10, 11, 12, 13, 14]
    # the target disagrees at the first draft: only its own token is kept
    ts = np.array([[5, 2, 3, 4, 77]], np.int32)
    r = oracle.accept(topo.parent, K, tok, ts, lens)
    assert r["accept_len"][0] == 1 and list(r["path"][0]) == [0, -1, -1, -1, -1]
    assert r["next_tok"][0] == 5 and list(r["compact_src"][0]) == [10, -1, -1, -1, -1]


def _random_tree_case(seed, B, topo, V):
    rng = np.random.default_rng(seed)
    tok = np.stack([rng.choice(V, topo.n, replace=False) for _ in range(B)]).astype(np.int32)
    logits = rng.standard_normal((B, topo.n, V)).astype(np.float32)
    return tok, logits


def test_accept_is_lossless_and_maximal():
    topo = product_order_tree((4, 2, 2, 1), 16)
    B, V, K = 300, 64, 4
    tok, logits = _random_tree_case(3, B, topo, V)
    plant(logits, topo, tok, (0.8, 0.65, 0.5, 0.4), seed=4)
    ts = oracle.argmax(logits)
    r = oracle.accept(topo.parent, K, tok, ts, np.zeros(B, np.int32))
    for b in range(B):
        A = r["accept_len"][b]
        path = r["path"][b]
        assert path[0] == 0 and all(p == -1 for p in path[A:])
        for j in range(1, A):
            assert topo.parent[path[j]] == path[j - 1]
            assert tok[b, path[j]] == ts[b, path[j - 1]]  # every accepted draft is the target's own choice
        last = path[A - 1]
        for c in range(topo.n):
            if topo.parent[c] == last:
                assert tok[b, c] != ts[b, last]  # nothing accepted beyond
        assert r["next_tok"][b] == ts[b, last]


def test_compaction_moves_exactly_the_accepted_slots():
    B, Hkv, hd, K = 2, 3, 8, 4
    Lcap = 40
    Kc = synth.normal(40, 1, (B, Hkv, Lcap, hd), 1.0, "bf16")
    Vc = synth.normal(41, 1, (B, Hkv, Lcap, hd), 1.0, "bf16")
    lens = np.array([7, 20], np.int32)
    acc = np.array([4, 1], np.int32)
    # request 0's path reads slot L+2 for j=1 and writes it for j=2 (overlap)
    path = np.array([[0, 2, 5, 9, -1], [0, -1, -1, -1, -1]], np.int32)
    K2, V2, l2 = oracle.compact(Kc, Vc, lens, acc, path, K)
    assert list(l2) == [11, 21]
    for b in range(B):
        L = lens[b]
        for X, X2 in ((Kc, K2), (Vc, V2)):
            assert np.array_equal(X2[b, :, :L], X[b, :, :L])
            for j in range(acc[b]):
                assert np.array_equal(X2[b, :, L + j], X[b, :, L + path[b, j]])
            assert np.array_equal(X2[b, :, L + acc[b]:], X[b, :, L + acc[b]:])


# -------------------------------------------- expected accepted length (E)

@pytest.mark.parametrize("row", [0, 1, 2])
def test_planted_acceptance_reproduces_page_table(row):
    """The mean accepted length over planted steps reproduces the page's E.

    Each request's accept length is produced by the oracle's argmax + accept
    on logits planted with per-depth acceptance a; its mean must match the
    E printed in the acceptance table, and E / cost its printed speedup.
    """
    g = golden("acceptance_table.json")["rows"][row]
    a = g["a"]
    K = 4
    topo = product_order_tree((4, 2, 2, 1), 16) if "tree" in g["name"] else chain(K)
    B, V = 20000, 48
    tok, logits = _random_tree_case(100 + row, B, topo, V)
    plant(logits, topo, tok, a, seed=200 + row)
    ts = oracle.argmax(logits)
    acc = oracle.accept(topo.parent, K, tok, ts, np.zeros(B, np.int32))["accept_len"]
    # distribution of the accepted length: P(len = j + 1) = a_1..a_j (1 - a_{j+1})
    p = []
    run = 1.0
    for j in range(K + 1):
        p.append(run * (1 - a[j]) if j < K else run)
        if j < K:
            run *= a[j]
    p = np.array(p)
    mean_model = float(np.sum(p * np.arange(1, K + 2)))
    var_model = float(np.sum(p * np.arange(1, K + 2) ** 2)) - mean_model ** 2
    tol = 4 * math.sqrt(var_model / B) + 0.005  # sampling + the page's rounding
    emp = float(acc.mean())
    assert abs(emp - g["E"]) < tol, (emp, g["E"], tol)
    counts = np.bincount(acc, minlength=K + 2)[1:]
    chi2 = float(np.sum((counts - B * p) ** 2 / (B * p)))
    assert chi2 < 20.5  # chi-square, 4 dof, p ~ 4e-4
    if "Medusa" in g["name"]:
        # cost = 1 + heads' bytes / target's bytes; the page prints E / cost
        hp = golden("head_params.json")
        cost = 1 + hp["heads"] * oracle.head_weight_elems(hp["d"], hp["d"], hp["V"]) * 2 / (hp["target_bytes_GB"] * 1e9)
        assert round(cost, 3) == g["cost"]
        assert abs(emp / cost - g["speedup"]) < tol / cost + 0.006


def test_planted_hidden_states_reproduce_page_table():
    """Verification through the target's LM head: hidden states planted with
    a = (0.80, 0.65, 0.50, 0.40) give, through the oracle's LM-head argmax and
    acceptance, the mean accepted length of the page's tree row (E = 2.68)."""
    g = golden("acceptance_table.json")["rows"][2]
    a, K = g["a"], 4
    topo = product_order_tree((4, 2, 2, 1), 16)
    B, V, d = 2000, 512, 64
    tok, _ = _random_tree_case(300, B, topo, V)
    Wt = synth.normal(301, 1, (V, d), 1 / math.sqrt(d), "f32")
    Ht = synth.normal(301, 2, (B, topo.n, d), 1.0, "f32")
    plant_hidden(Ht, Wt, topo, tok, a, seed=302)
    ts, _, margin = oracle.target_argmax(Ht.reshape(B * topo.n, d), Wt)
    acc = oracle.accept(topo.parent, K, tok, ts.reshape(B, topo.n), np.zeros(B, np.int32))["accept_len"]
    p, run = [], 1.0
    for j in range(K + 1):
        p.append(run * (1 - a[j]) if j < K else run)
        if j < K:
            run *= a[j]
    p = np.array(p)
    mean_model = float(np.sum(p * np.arange(1, K + 2)))
    var_model = float(np.sum(p * np.arange(1, K + 2) ** 2)) - mean_model ** 2
    tol = 4 * math.sqrt(var_model / B) + 0.005
    assert abs(float(acc.mean()) - g["E"]) < tol, (float(acc.mean()), g["E"], tol)
    counts = np.bincount(acc, minlength=K + 2)[1:]
    assert float(np.sum((counts - B * p) ** 2 / (B * p))) < 20.5
