"""GPU parity of the target's LM head with a fused argmax (md_target_argmax)
and of acceptance fed with the target's tokens (md_tree_accept_tokens).

The argmax follows the margin rule with k = 1: where the oracle's top two
logits are more than tau apart the token must match, otherwise the GPU's
token must be within tau of the maximum. Values follow the relative
tolerance. Sizes cover the GEMV path (float32, few rows), the MFMA path
(bf16, ragged rows and vocabulary tiles, more than 1,024 partial lists; 65 to
128 rows in one register-streamed tile) and the 70B-shaped LM head over a
64-node tree.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from synth.topology import product_order_tree
from synth.workloads import plant

from _helpers import TAU, TOL, from_dev, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ("f32 gemv R=16", "f32", 16, 256, 4096),
    ("bf16 gemv R=5", "bf16", 5, 512, 5003),
    ("bf16 mfma R=64", "bf16", 64, 512, 5003),
    ("bf16 mfma R=100 one tile", "bf16", 100, 256, 4099),
    ("bf16 mfma R=128 one tile", "bf16", 128, 128, 2053),
    ("bf16 mfma R=72 fewer K steps than the ring", "bf16", 72, 128, 3001),
    ("bf16 mfma R=88 six column blocks, fewer K steps than the ring", "bf16", 88, 128, 3001),
    ("bf16 mfma R=130 ragged", "bf16", 130, 256, 3001),
    ("bf16 mfma many lists R=9", "bf16", 9, 128, 140001),
    ("70B-shaped LM head, 64 nodes", "bf16", 64, 8192, 128256),
]


def gpu_argmax(dtype, R, d, V, H, Wt, op=False):
    import torch

    import medusa_draft_heads_amd as md

    dt = md.MD_F32 if dtype == "f32" else md.MD_BF16
    tok = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    val = torch.empty(R, dtype=torch.float32, device="cuda")
    ws = torch.empty(md.md_target_argmax_workspace_bytes(dt, R, d, V), dtype=torch.uint8, device="cuda")
    Wt_dev = to_dev(Wt)
    Wt_op = md.operand_order(Wt_dev) if op else None
    md.md_target_argmax(dt, R, d, V, to_dev(H), Wt_dev, tok, val, ws, Wt_op=Wt_op)
    torch.cuda.synchronize()
    return from_dev(tok), from_dev(val)


OP_CASES = [
    ("bf16 operand order R=1 (GEMV, copy unused)", "bf16", 1, 512, 5003, True),
    ("bf16 operand order R=2", "bf16", 2, 512, 5003, True),
    ("bf16 operand order R=7", "bf16", 7, 256, 4099, True),
    ("bf16 operand order R=64", "bf16", 64, 512, 5003, True),
    ("bf16 operand order R=80 five full column blocks", "bf16", 80, 256, 4099, True),
    ("bf16 operand order R=81 one column of a sixth block", "bf16", 81, 512, 5003, True),
    ("bf16 operand order R=100 one tile", "bf16", 100, 256, 4099, True),
    ("bf16 operand order R=128 one tile", "bf16", 128, 128, 2053, True),
    ("bf16 operand order R=130 row-major kernel", "bf16", 130, 256, 3001, True),
    ("bf16 operand order many lists R=9", "bf16", 9, 128, 140001, True),
    ("70B-shaped LM head in operand order, 64 nodes", "bf16", 64, 8192, 128256, True),
]


@pytest.mark.parametrize("case", [c + (False,) for c in CASES] + OP_CASES,
                         ids=[c[0] for c in CASES] + [c[0] for c in OP_CASES])
def test_target_argmax(case):
    """With an operand-order copy of the LM head, 2 to 128 rows run the few-row matrix-core kernels
    on it (more rows keep the row-major kernel); from 8 rows the result is the row-major run's, bit
    for bit."""
    name, dtype, R, d, V, op = case
    seed = R + d
    Wt = synth.normal(seed, 1, (V, d), 1 / math.sqrt(d), dtype)
    H = synth.normal(seed, 2, (R, d), 1.0, dtype)
    tok, val = gpu_argmax(dtype, R, d, V, H, Wt, op)
    rtok, rval, margin = oracle.target_argmax(H, Wt)
    tau, tol = TAU[dtype], TOL[dtype]
    ties = 0
    Hf = synth.bf16_to_f32(H).astype(np.float64) if dtype == "bf16" else H.astype(np.float64)
    for r in range(R):
        if margin[r] > tau:
            assert tok[r] == rtok[r], (name, r, tok[r], rtok[r], margin[r])
        else:
            ties += 1
            w = synth.bf16_to_f32(Wt[tok[r]]).astype(np.float64) if dtype == "bf16" else Wt[tok[r]].astype(np.float64)
            assert rval[r] - float(w @ Hf[r]) <= tau
    assert np.max(np.abs(val - rval)) <= tol * np.max(np.abs(rval))
    # bit-identical on a second call
    tok2, val2 = gpu_argmax(dtype, R, d, V, H, Wt, op)
    assert np.array_equal(tok, tok2) and np.array_equal(val.view(np.uint32), val2.view(np.uint32))
    if op and R >= 8:
        tok3, val3 = gpu_argmax(dtype, R, d, V, H, Wt)
        assert np.array_equal(tok, tok3) and np.array_equal(val.view(np.uint32), val3.view(np.uint32))
    print("%s: near ties %d of %d" % (name, ties, R))


def test_target_argmax_lowest_index_on_ties():
    # an identity head over d = V makes the logits the hidden state: rows with
    # equal maxima must pick the lower index on both paths
    d = V = 256
    for dtype, R in (("f32", 3), ("bf16", 8)):
        Wt = np.eye(d, dtype=np.float32)
        H = synth.normal(4, 3, (R, d), 1.0, "f32")
        H[:, 17] = H[:, 200] = np.float32(8.0)
        if dtype == "bf16":
            Wt, H = synth.f32_to_bf16(Wt), synth.f32_to_bf16(H)
        tok, val = gpu_argmax(dtype, R, d, V, H, Wt)
        assert np.all(tok == 17) and np.all(val == 8.0), (dtype, tok)


ACCEPT_CASES = [
    ("tiny f32", "f32", ((4, 2, 2, 1), 16), 4, 1, 4096, 2, 64, [128], 144),
    ("64-node bf16 batch 5", "bf16", ((10, 4, 2, 1), 64), 4, 5, 3001, 8, 128, [0, 5, 100, 1000, 33], 1064),
    ("tree past capacity", "bf16", ((4, 2, 2, 1), 16), 4, 3, 500, 2, 64, [4, 30, -2], 40),
]


@pytest.mark.parametrize("case", ACCEPT_CASES, ids=[c[0] for c in ACCEPT_CASES])
def test_tree_accept_tokens(case):
    """Acceptance and compaction from given target tokens equal the oracle's, bit for bit."""
    import torch

    import medusa_draft_heads_amd as md

    name, dtype, (kph, N), K, B, V, Hkv, hd, lens, Lcap = case
    topo = product_order_tree(kph, N)
    seed = len(name) + 40
    rng = np.random.default_rng(seed)
    tok = np.stack([rng.choice(V, N, replace=False) for _ in range(B)]).astype(np.int32)
    logits = synth.normal(seed, 9, (B, N, V), 1.0, "f32")
    plant(logits, topo, tok, (0.8, 0.65, 0.5, 0.4), seed=seed)
    ts = oracle.argmax(logits)  # the target's tokens, from the oracle
    Kc = synth.normal(seed, 2, (B, Hkv, Lcap, hd), 1.0, dtype)
    Vc = synth.normal(seed, 3, (B, Hkv, Lcap, hd), 1.0, dtype)
    lens = np.asarray(lens, np.int32)
    ref = oracle.accept(topo.parent, K, tok, ts, lens)
    valid = (lens >= 0) & (lens + N <= Lcap)
    rK, rV, rl = oracle.compact(Kc, Vc, lens, np.where(valid, ref["accept_len"], 0), ref["path"], K)
    dt = md.MD_F32 if dtype == "f32" else md.MD_BF16
    kc, vc, ld = to_dev(Kc), to_dev(Vc), to_dev(lens)
    outs = {k: torch.empty(*s, dtype=torch.int32, device="cuda") for k, s in
            (("accept_len", (B,)), ("path", (B, K + 1)), ("next_tok", (B,)), ("compact_src", (B, K + 1)))}
    md.md_tree_accept_tokens(md.make_tree(topo.parent, topo.rank), dt, B, K, Hkv, hd, Lcap, to_dev(ts), to_dev(tok),
                             kc, vc, ld, outs["accept_len"], outs["path"], outs["next_tok"], outs["compact_src"])
    torch.cuda.synchronize()
    got = {k: from_dev(v) for k, v in outs.items()}
    for b in range(B):
        if valid[b]:
            for key in ("accept_len", "next_tok", "path", "compact_src"):
                assert np.array_equal(got[key][b], ref[key][b]), (key, b, got[key][b], ref[key][b])
        else:
            assert got["accept_len"][b] == 0 and got["next_tok"][b] == -1
    assert np.array_equal(from_dev(kc), rK) and np.array_equal(from_dev(vc), rV)
    assert np.array_equal(from_dev(ld), rl)
    print(name, "accept_len", list(got["accept_len"]))
