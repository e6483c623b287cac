"""md_tree_attention_noalloc, the tree attention for callers that cannot
allocate, against md_tree_attention with a caller workspace: the same
kernels, so the outputs must be equal bit for bit, and both within the
tolerance of the oracle. Two calls in a row (the second smaller, so it runs
on scratch that still holds the first call's partial rows), then a float32
call."""
import numpy as np
import pytest

import oracle
import synth
from synth.topology import product_order_tree

from _helpers import TOL, from_dev, rel_err, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # name, dtype, B, topology, Hq, Hkv, hd, lens
    ("70B-shaped bf16", "bf16", 1, ((10, 4, 2, 1), 64), 64, 8, 128, [4096]),
    ("ragged bf16, smaller", "bf16", 3, ((4, 2, 2, 1), 16), 8, 2, 128, [0, 1, 777]),
    ("tiny f32", "f32", 1, ((4, 2, 2, 1), 16), 4, 2, 64, [128]),
]


def _attend(md, noalloc, tree, dt, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, out_dtype, N):
    import torch

    out = torch.empty(B, N, Hq, hd, dtype=out_dtype, device="cuda")
    if noalloc:
        md.md_tree_attention_noalloc(tree, dt, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, 1.0 / np.sqrt(hd), out)
    else:
        ws = torch.empty(md.md_attention_workspace_bytes(dt, B, N, Hq, Hkv, hd, max_len), dtype=torch.uint8,
                         device="cuda")
        md.md_tree_attention(tree, dt, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, 1.0 / np.sqrt(hd), out, ws)
    torch.cuda.synchronize()
    return from_dev(out)


def test_attention_noalloc_matches_workspace_call():
    import torch

    import medusa_draft_heads_amd as md

    for i, (name, dtype, B, (kph, N), Hq, Hkv, hd, lens) in enumerate(CASES):
        topo = product_order_tree(kph, N)
        lens = np.asarray(lens, np.int32)
        max_len = int(lens.max())
        Lcap = max_len + N + 3
        seed = 900 + i
        q = synth.normal(seed, 1, (B, N, Hq, hd), 1.0, dtype)
        Kc = synth.normal(seed, 2, (B, Hkv, Lcap, hd), 1.0, dtype)
        Vc = synth.normal(seed, 3, (B, Hkv, Lcap, hd), 1.0, dtype)
        dt = md.MD_F32 if dtype == "f32" else md.MD_BF16
        out_dtype = torch.float32 if dtype == "f32" else torch.bfloat16
        need = md.md_attention_workspace_bytes(dt, B, N, Hq, Hkv, hd, max_len)
        assert need <= md.md_tree_attention_noalloc_max_bytes(), (name, need)
        args = (md.make_tree(topo.parent, topo.rank), dt, B, Hq, Hkv, hd, Lcap, max_len, to_dev(q), to_dev(Kc),
                to_dev(Vc), to_dev(lens), out_dtype, N)
        got_na = _attend(md, True, *args)
        got_ws = _attend(md, False, *args)
        assert np.array_equal(got_na.view(np.uint8), got_ws.view(np.uint8)), "%s: outputs differ" % name
        ref = oracle.tree_attention(topo.parent, q, Kc, Vc, lens)
        g = got_na.astype(np.float64) if dtype == "f32" else synth.bf16_to_f32(got_na).astype(np.float64)
        err = rel_err(g, ref)
        print("%s (scratch %d bytes): bit-equal to the workspace call, relative error %.3g" % (name, need, err))
        assert err <= TOL[dtype]
