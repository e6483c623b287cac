"""GPU parity of md_tree_build, md_tree_attention and md_tree_accept.

Each stage is fed the oracle's own upstream values, so every integer output
(tree tokens and positions, accepted lengths, paths, next tokens, compaction
indices, the moved cache bytes, the new lengths) must match bit for bit;
attention outputs match within the relative tolerance.
"""
import zlib
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from synth.topology import chain, product_order_tree
from synth.workloads import LLAMA8B, LLAMA70B, LLAMA70B_B8, TINY_F32, HYDRA_B4, Workload, plant, step_inputs

from _helpers import TOL, from_dev, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _md():
    import medusa_draft_heads_amd as md

    return md


# ------------------------------------------------------------------ tree

@pytest.mark.parametrize("k_per_head,N,B,M", [((4, 2, 2, 1), 16, 1, 1), ((10, 4, 2, 1), 64, 3, 5),
                                              ((1, 1, 1, 1), 5, 2, 2), ((3,), 1, 2, 2)])
def test_tree_build_medusa(k_per_head, N, B, M):
    import torch

    md = _md()
    K = len(k_per_head)
    topo = product_order_tree(k_per_head, N)
    kmax = max(k_per_head)
    rng = np.random.default_rng(N + B)
    lists = rng.integers(0, 128256, size=(M, K, kmax)).astype(np.int32)
    src = rng.integers(0, M, size=B).astype(np.int32)
    root = rng.integers(0, 128256, size=B).astype(np.int32)
    lens = rng.integers(0, 5000, size=B).astype(np.int32)
    ref_tok, ref_pos = oracle.tree_tokens_medusa(topo.parent, topo.rank, lists, src, root, lens)
    tok = torch.empty(B, N, dtype=torch.int32, device="cuda")
    pos = torch.empty(B, N, dtype=torch.int32, device="cuda")
    md.md_tree_build(md.make_tree(topo.parent, topo.rank), 0, B, M, K, kmax, 0, to_dev(lists), to_dev(src),
                     to_dev(root), to_dev(lens), tok, pos)
    assert np.array_equal(from_dev(tok), ref_tok) and np.array_equal(from_dev(pos), ref_pos)


def test_tree_build_bad_source_row_gives_no_tokens():
    import torch

    md = _md()
    topo = product_order_tree((4, 2, 2, 1), 16)
    lists = np.zeros((2, 4, 4), np.int32)
    tok = torch.empty(2, 16, dtype=torch.int32, device="cuda")
    pos = torch.empty(2, 16, dtype=torch.int32, device="cuda")
    md.md_tree_build(md.make_tree(topo.parent, topo.rank), 0, 2, 2, 4, 4, 0, to_dev(lists),
                     to_dev(np.array([5, -1], np.int32)), to_dev(np.array([7, 8], np.int32)),
                     to_dev(np.array([0, 3], np.int32)), tok, pos)
    t = from_dev(tok)
    assert list(t[:, 0]) == [7, 8] and np.all(t[:, 1:] == -1)


# ------------------------------------------------------------- attention

ATTN_CASES = [
    # name, dtype, B, topology, Hq, Hkv, hd, lens
    ("tiny f32", "f32", 1, ((4, 2, 2, 1), 16), 4, 2, 64, [128]),
    ("ragged bf16", "bf16", 3, ((4, 2, 2, 1), 16), 8, 2, 128, [0, 1, 777]),
    ("chain bf16 hd64", "bf16", 2, ((1, 1, 1, 1), 5), 6, 3, 64, [100, 65]),
    ("root only f32", "f32", 2, ((1,), 1), 2, 1, 64, [0, 3]),
    ("8B-shaped bf16", "bf16", 1, ((10, 4, 2, 1), 64), 32, 8, 128, [2048]),
    ("70B-shaped bf16", "bf16", 1, ((10, 4, 2, 1), 64), 64, 8, 128, [4096]),
    ("Hydra-shaped bf16 batch 4", "bf16", 4, ((10, 4, 2, 1), 64), 32, 8, 128, [8192] * 4),
    # one query head per kv head: few query tiles, so the keys split into
    # 26 ranges (the combine merges them 8 at a time, then a partial 2)
    ("many key ranges bf16", "bf16", 1, ((10, 4, 2, 1), 64), 8, 8, 128, [4096]),
    # 32 ranges; the second request's 21 keys leave all ranges past the first empty
    ("many ranges ragged bf16 hd64", "bf16", 2, ((4, 2, 2, 1), 16), 4, 4, 64, [3000, 5]),
]


def case_seed(name: str) -> int:
    """A seed fixed by the case's name (the same in every process)."""
    return zlib.crc32(name.encode()) % 1000


def run_attention(dtype, B, topo, Hq, Hkv, hd, lens, seed, max_len=None, Lcap=None, v_scale=None):
    import torch

    md = _md()
    N = topo.n
    lens = np.asarray(lens, np.int32)
    max_len = int(lens.max()) if max_len is None else max_len
    Lcap = max_len + N + 3 if Lcap is None else Lcap
    q = synth.normal(seed, 1, (B, N, Hq, hd), 1.0, dtype)
    Kc = synth.normal(seed, 2, (B, Hkv, Lcap, hd), 1.0, dtype)
    Vc = synth.normal(seed, 3, (B, Hkv, Lcap, hd), 1.0, dtype)
    if v_scale is not None:  # a power of two: the stored values stay exact
        Vc = (synth.bf16_to_f32(Vc) * np.float32(v_scale)).astype(np.float32)
        Vc = synth.f32_to_bf16(Vc) if dtype == "bf16" else Vc
    dt = md.MD_F32 if dtype == "f32" else md.MD_BF16
    out = torch.empty(B, N, Hq, hd, dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
    ws = torch.empty(md.md_attention_workspace_bytes(dt, B, N, Hq, Hkv, hd, max_len), dtype=torch.uint8, device="cuda")
    md.md_tree_attention(md.make_tree(topo.parent, topo.rank), dt, B, Hq, Hkv, hd, Lcap, max_len, to_dev(q),
                         to_dev(Kc), to_dev(Vc), to_dev(lens), 1.0 / np.sqrt(hd), out, ws)
    torch.cuda.synchronize()
    got = from_dev(out)
    ref = oracle.tree_attention(topo.parent, q, Kc, Vc, lens)
    return got, ref


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_tree_attention(case):
    name, dtype, B, (kph, N), Hq, Hkv, hd, lens = case
    topo = product_order_tree(kph, N)
    seed = case_seed(name)
    got, ref = run_attention(dtype, B, topo, Hq, Hkv, hd, lens, seed=seed)
    g = got.astype(np.float64) if dtype == "f32" else synth.bf16_to_f32(got).astype(np.float64)
    err = rel_err(g, ref)
    print("%s (seed %d): relative error %.3g" % (name, seed, err))
    assert err <= TOL[dtype], "%s (seed %d): relative error %.3g" % (name, seed, err)


@pytest.mark.parametrize("v_scale", [2.0 ** 17, 2.0 ** -20, 2.0 ** 60], ids=["V~1e5", "V~1e-6", "V~1e18"])
def test_tree_attention_value_range(v_scale):
    """bf16 values far outside the 16-bit float range of the partial rows the key ranges hand to the
    combine (up to ~4e5, ~4e-6 and ~4e18 with V ~ N(0, 1) scaled): every output row within the
    tolerance of that row's own largest entry."""
    topo = product_order_tree((4, 2, 2, 1), 16)
    lens = [0, 300, 2000]
    got, ref = run_attention("bf16", 3, topo, 8, 2, 128, lens, seed=17, v_scale=v_scale)
    g = synth.bf16_to_f32(got).astype(np.float64)
    assert np.all(np.isfinite(g))
    num = np.max(np.abs(g - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    worst = float(np.max(num / den))
    print("V scaled by %g: worst row relative error %.3g" % (v_scale, worst))
    assert worst <= TOL["bf16"]


def test_tree_attention_batch8_ragged_full_size():
    wl = LLAMA70B_B8
    x = step_inputs(wl, 88)
    topo = wl.topology()
    lens = x["lens"]
    got, ref = run_attention("bf16", wl.B, topo, wl.Hq, wl.Hkv, wl.hd, lens, seed=88, max_len=wl.L_max,
                             Lcap=wl.Lcap)
    err = rel_err(synth.bf16_to_f32(got).astype(np.float64), ref)
    print("batch 8 ragged (lens %s): relative error %.3g" % (list(lens), err))
    assert err <= TOL["bf16"]


# ----------------------------------------------------------------- accept

def run_accept(dtype, topo, K, B, V, Hkv, hd, lens, Lcap, seed, a=(0.8, 0.65, 0.5, 0.4), tok=None, logits=None):
    import torch

    md = _md()
    N = topo.n
    rng = np.random.default_rng(seed)
    if tok is None:
        tok = np.stack([rng.choice(V, N, replace=False) for _ in range(B)]).astype(np.int32)
    if logits is None:
        logits = synth.normal(seed, 9, (B, N, V), 1.0, "f32")
        plant(logits, topo, tok, a, seed=seed)
    Kc = synth.normal(seed, 2, (B, Hkv, Lcap, hd), 1.0, dtype)
    Vc = synth.normal(seed, 3, (B, Hkv, Lcap, hd), 1.0, dtype)
    lens = np.asarray(lens, np.int32)
    ref = oracle.accept(topo.parent, K, tok, oracle.argmax(logits), lens)
    valid = (lens >= 0) & (lens + N <= Lcap)
    rK, rV, rl = oracle.compact(Kc, Vc, lens, np.where(valid, ref["accept_len"], 0), ref["path"], K)
    dt = md.MD_F32 if dtype == "f32" else md.MD_BF16
    kc, vc, ld = to_dev(Kc), to_dev(Vc), to_dev(lens)
    outs = {k: torch.empty(*s, dtype=torch.int32, device="cuda") for k, s in
            (("accept_len", (B,)), ("path", (B, K + 1)), ("next_tok", (B,)), ("compact_src", (B, K + 1)))}
    ws = torch.empty(md.md_accept_workspace_bytes(B, N, V), dtype=torch.uint8, device="cuda")
    md.md_tree_accept(md.make_tree(topo.parent, topo.rank), dt, B, K, V, Hkv, hd, Lcap, to_dev(logits), to_dev(tok),
                      kc, vc, ld, outs["accept_len"], outs["path"], outs["next_tok"], outs["compact_src"], ws)
    torch.cuda.synchronize()
    got = {k: from_dev(v) for k, v in outs.items()}
    for b in range(B):
        if valid[b]:
            for key in ("accept_len", "next_tok"):
                assert got[key][b] == ref[key][b], (key, b, got[key][b], ref[key][b])
            for key in ("path", "compact_src"):
                assert np.array_equal(got[key][b], ref[key][b]), (key, b, got[key][b], ref[key][b])
        else:
            # a request whose tree does not fit the cache is left untouched
            assert got["accept_len"][b] == 0 and got["next_tok"][b] == -1
            assert np.all(got["path"][b] == -1) and np.all(got["compact_src"][b] == -1)
    assert np.array_equal(from_dev(kc), rK) and np.array_equal(from_dev(vc), rV)
    assert np.array_equal(from_dev(ld), rl)
    return got, ref


ACCEPT_CASES = [
    ("tiny f32", "f32", ((4, 2, 2, 1), 16), 4, 1, 4096, 2, 64, [128], 144),
    ("64-node bf16 batch 5", "bf16", ((10, 4, 2, 1), 64), 4, 5, 3001, 8, 128, [0, 5, 100, 1000, 33], 1064),
    ("chain bf16", "bf16", ((1, 1, 1, 1), 5), 4, 3, 777, 4, 128, [10, 0, 7], 20),
    ("root only", "f32", ((2,), 1), 1, 2, 100, 1, 64, [3, 4], 8),
    ("70B-shaped", "bf16", ((10, 4, 2, 1), 64), 4, 1, 128256, 8, 128, [4096], 4160),
    ("70B-shaped batch 8 (512 rows)", "bf16", ((10, 4, 2, 1), 64), 4, 8, 128256, 8, 128,
     [1024, 4096, 2000, 3333, 1500, 4000, 1025, 2718], 4160),
    ("tree past capacity", "bf16", ((4, 2, 2, 1), 16), 4, 3, 500, 2, 64, [4, 30, -2], 40),
]


@pytest.mark.parametrize("case", ACCEPT_CASES, ids=[c[0] for c in ACCEPT_CASES])
def test_tree_accept(case):
    name, dtype, (kph, N), K, B, V, Hkv, hd, lens, Lcap = case
    topo = product_order_tree(kph, N)
    got, ref = run_accept(dtype, topo, K, B, V, Hkv, hd, lens, Lcap, seed=len(name))
    print(name, "accept_len", list(got["accept_len"]))


def test_accept_full_chain_and_overlap():
    # a = 1 plants every depth: the whole chain is accepted; the 64-node tree
    # case accepts a deep branch whose source slots overlap its destinations
    topo = chain(4)
    got, _ = run_accept("bf16", topo, 4, 2, 1000, 2, 64, [9, 0], 20, seed=5, a=(1, 1, 1, 1))
    assert list(got["accept_len"]) == [5, 5]
    topo = product_order_tree((10, 4, 2, 1), 64)
    got, _ = run_accept("bf16", topo, 4, 16, 2000, 2, 128, [50] * 16, 120, seed=6, a=(1, 1, 1, 1))
    assert np.all(got["accept_len"] == 5)
    assert any(got["path"][b][1] != 1 for b in range(16))  # a non-identity move happened


def test_accept_argmax_ties_take_lowest_index():
    topo = chain(2)
    V = 64
    logits = np.zeros((1, 3, V), np.float32)  # every row all ties -> argmax 0
    tok = np.array([[5, 0, 7]], np.int32)  # node 1 matches t*(root) = 0; node 2 would need t*(1) = 7
    got, ref = run_accept("f32", topo, 2, 1, V, 1, 64, [2], 8, seed=1, tok=tok, logits=logits)
    assert got["accept_len"][0] == 2 and got["next_tok"][0] == 0


def test_accept_argmax_512_rows_ties_across_halves():
    """Batch 8 x 64 nodes = 512 rows of the full 128,256-entry vocabulary (the batch-8 verification
    shape, where the argmax splits each row into chunks). Every row's two largest logits lie one in
    each half of the row: equal (the lower index must win) or the upper one larger by 0.5 (the
    larger must win). A node's first child carries its parent's target choice and its second child
    the parent's other planted index, so the accepted branch is the first-child chain to depth 4,
    and a wrong choice at any row on it changes the path, the length or the next token."""
    topo = product_order_tree((10, 4, 2, 1), 64)
    B, V, N = 8, 128256, topo.n
    rng = np.random.default_rng(11)
    half = V // 2
    i0 = rng.integers(0, half, size=(B, N))
    i1 = rng.integers(half, V, size=(B, N))
    bigger = rng.random((B, N)) < 0.5
    logits = np.zeros((B, N, V), np.float32)
    bi, ni = np.meshgrid(np.arange(B), np.arange(N), indexing="ij")
    logits[bi, ni, i0] = 10.0
    logits[bi, ni, i1] = np.where(bigger, 10.5, 10.0).astype(np.float32)
    tstar = np.where(bigger, i1, i0)
    other = np.where(bigger, i0, i1)
    tok = np.zeros((B, N), np.int32)
    for b in range(B):
        tok[b, 0] = 7
        for n in range(1, N):
            p, r = topo.parent[n], topo.rank[n]
            tok[b, n] = tstar[b, p] if r == 0 else (other[b, p] if r == 1 else (tstar[b, p] + r) % V)
    got, ref = run_accept("bf16", topo, 4, B, V, 8, 128, [100] * B, 200, seed=12, tok=tok, logits=logits)
    assert np.all(ref["accept_len"] == 5) and np.all(got["accept_len"] == 5)
    deepest = got["path"][:, 4]
    assert np.array_equal(got["next_tok"], tstar[np.arange(B), deepest])
