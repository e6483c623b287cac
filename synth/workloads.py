"""The decode-step workloads and their seeded synthetic tensors.

Shapes follow the pages' running example (Medusa heads versus separate draft
model: Llama 3 vocabulary V = 128,256; Llama 3.3 70B hidden size d = 8,192;
four heads) plus an 8B-shaped, a batch-8 and a Hydra variant. Every tensor is
drawn from its own Philox stream (see ``synth.c``); per-step tensors fold the
step index into the stream so a bench can rotate independent input sets.

Nothing here computes the decode step. ``plant`` builds verification logits
with a prescribed per-depth acceptance from the tree tokens it is handed;
``plant_hidden`` does the same in the target's hidden states when the
verification runs through the target's LM head.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from . import normal, randint, u32, uniform01
from .topology import Topology, product_order_tree

# stream ids (low byte); the step index is folded in above it
S_H, S_W, S_B, S_U, S_E, S_Q, S_K, S_V, S_LOGITS, S_ROOT, S_LENS, S_PLANT, S_SRC, S_WT, S_HT, S_ALT = range(1, 17)
S_DRAFTW, S_UW, S_GW = range(17, 20)  # random words of sampled decoding


def stream(sid: int, step: int = 0) -> int:
    return (step << 8) | sid


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "medusa" | "hydra"
    B: int
    d: int
    V: int
    K: int
    dtype: str  # "f32" | "bf16"
    topk: Tuple[int, ...]
    N: int
    Hq: int
    Hkv: int
    hd: int
    L: Optional[int] = None  # every request's cached length
    L_range: Optional[Tuple[int, int]] = None  # or uniform on [lo, hi] per request
    a: Tuple[float, ...] = (0.80, 0.65, 0.50, 0.40)
    rows_per_request: int = 1  # 1: heads on the last hidden state; N: on every tree node
    bias_zero: bool = False
    chain: bool = False
    shared_u: bool = False  # one vocabulary projection U [V, d] for every head
    target_head: bool = False  # verify from the target's hidden states Ht [B, N, d] through its LM head Wt [V, d]
    # "greedy": argmax matching; "sampled": drafts drawn from the heads and
    # rejection-sampling verification; "typical": top-k drafts and typical acceptance
    verify: str = "greedy"
    temperature: float = 1.0
    eps: float = 0.09    # typical acceptance: threshold min(eps, delta exp(-H))
    delta: float = 0.3

    @property
    def kmax(self) -> int:
        return max(self.topk)

    @property
    def L_max(self) -> int:
        return self.L if self.L is not None else self.L_range[1]

    @property
    def Lcap(self) -> int:
        return self.L_max + self.N

    @property
    def din(self) -> int:
        return 2 * self.d if self.kind == "hydra" else self.d

    @property
    def M(self) -> int:
        return self.B * self.rows_per_request

    def topology(self) -> Topology:
        return product_order_tree(self.topk, self.N)

    # ---- byte accounting of the weights the heads read (per head / total) ----
    def head_params(self) -> Dict[str, int]:
        res = self.d * self.din + self.d
        voc = self.d * self.V
        return {"residual": res, "vocab": voc, "per_head": res + voc, "total": self.K * (res + voc)}


TINY_F32 = Workload("tiny f32: d=256 V=4096 K=4, 16-node tree, GQA 4/2 hd64, L=128", "medusa",
                    B=1, d=256, V=4096, K=4, dtype="f32", topk=(4, 2, 2, 1), N=16,
                    Hq=4, Hkv=2, hd=64, L=128, bias_zero=True)
LLAMA8B = Workload("8B-shaped bf16: d=4096 V=128256 K=4, 64-node tree, GQA 32/8 hd128, L=2048", "medusa",
                   B=1, d=4096, V=128256, K=4, dtype="bf16", topk=(10, 4, 2, 1), N=64,
                   Hq=32, Hkv=8, hd=128, L=2048)
LLAMA70B = Workload("70B-shaped bf16 heads, batch 1: d=8192 V=128256 K=4, 64-node tree, GQA 64/8 hd128, L=4096",
                    "medusa", B=1, d=8192, V=128256, K=4, dtype="bf16", topk=(10, 4, 2, 1), N=64,
                    Hq=64, Hkv=8, hd=128, L=4096)
LLAMA70B_CHAIN = replace(LLAMA70B, name="70B-shaped bf16 heads, batch 1, top-1 chain: N=5",
                         topk=(1, 1, 1, 1), N=5, a=(0.65, 0.50, 0.40, 0.35), chain=True)
LLAMA70B_B8 = Workload("70B-shaped bf16 heads, batch 8 over all 512 tree nodes: d=8192 V=128256, "
                       "GQA 64/8 hd128, L~U[1024,4096]", "medusa",
                       B=8, d=8192, V=128256, K=4, dtype="bf16", topk=(10, 4, 2, 1), N=64,
                       Hq=64, Hkv=8, hd=128, L_range=(1024, 4096), rows_per_request=64)
LLAMA70B_SHARED = replace(LLAMA70B, name="70B-shaped bf16 heads sharing one vocabulary projection, batch 1: "
                          "d=8192 V=128256 K=4, 64-node tree, GQA 64/8 hd128, L=4096", shared_u=True)
HYDRA_B4 = Workload("Hydra bf16, batch 4: d=4096 V=128256 K=4 sequential heads, GQA 32/8 hd128, L=8192",
                    "hydra", B=4, d=4096, V=128256, K=4, dtype="bf16", topk=(10, 4, 2, 1), N=64,
                    Hq=32, Hkv=8, hd=128, L=8192, a=(0.85, 0.75, 0.65, 0.55))

LLAMA70B_LMHEAD = replace(LLAMA70B, name="70B-shaped bf16 heads, batch 1, verified through the target's LM head "
                          "(128256 x 8192) with a fused argmax: d=8192 V=128256 K=4, 64-node tree, GQA 64/8 hd128, "
                          "L=4096", target_head=True)

LLAMA70B_SAMPLED = replace(LLAMA70B, name="70B-shaped bf16 heads, batch 1, sampled at T = 1: drafts drawn from "
                          "the heads, rejection-sampling verification: d=8192 V=128256 K=4, 64-node tree, GQA 64/8 "
                          "hd128, L=4096", verify="sampled")
LLAMA70B_TYPICAL = replace(LLAMA70B, name="70B-shaped bf16 heads, batch 1, typical acceptance at T = 1 (eps 0.09, "
                           "delta 0.3): d=8192 V=128256 K=4, 64-node tree, GQA 64/8 hd128, L=4096", verify="typical")
TINY_SAMPLED = replace(TINY_F32, name="tiny f32, sampled at T = 1", verify="sampled")
TINY_TYPICAL = replace(TINY_F32, name="tiny f32, typical acceptance at T = 1", verify="typical")

ALL = {"tiny": TINY_F32, "8b": LLAMA8B, "70b": LLAMA70B, "70b_chain": LLAMA70B_CHAIN,
       "70b_b8": LLAMA70B_B8, "hydra_b4": HYDRA_B4, "70b_shared": LLAMA70B_SHARED, "70b_lmhead": LLAMA70B_LMHEAD,
       "70b_sampled": LLAMA70B_SAMPLED, "70b_typical": LLAMA70B_TYPICAL, "tiny_sampled": TINY_SAMPLED,
       "tiny_typical": TINY_TYPICAL}


def weights(wl: Workload, seed: int, heads: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """W [K,d,din], b [K,d], U [K,V,d] ([V,d] when shared; it then equals head 0's U of the
    unshared workload) and E [V,d] for Hydra, all ~N(0, 1/d)."""
    std = 1.0 / np.sqrt(wl.d)
    out: Dict[str, np.ndarray] = {}
    out["W"] = normal(seed, stream(S_W), (wl.K, wl.d, wl.din), std, wl.dtype)
    if wl.bias_zero:
        out["b"] = np.zeros((wl.K, wl.d), dtype=np.float32 if wl.dtype == "f32" else np.uint16)
    else:
        out["b"] = normal(seed, stream(S_B), (wl.K, wl.d), std, wl.dtype)
    out["U"] = normal(seed, stream(S_U), ((wl.V, wl.d) if wl.shared_u else (wl.K, wl.V, wl.d)), std, wl.dtype)
    if wl.kind == "hydra":
        out["E"] = normal(seed, stream(S_E), (wl.V, wl.d), std, wl.dtype)
    if wl.target_head:
        out["Wt"] = normal(seed, stream(S_WT), (wl.V, wl.d), std, wl.dtype)
    return out


def step_inputs(wl: Workload, seed: int, step: int = 0) -> Dict[str, np.ndarray]:
    """Per-step tensors: hidden states, tree queries, KV cache, lengths, tokens, logits."""
    out: Dict[str, np.ndarray] = {}
    out["h"] = normal(seed, stream(S_H, step), (wl.M, wl.d), 1.0, wl.dtype)
    out["q"] = normal(seed, stream(S_Q, step), (wl.B, wl.N, wl.Hq, wl.hd), 1.0, wl.dtype)
    out["Kc"] = normal(seed, stream(S_K, step), (wl.B, wl.Hkv, wl.Lcap, wl.hd), 1.0, wl.dtype)
    out["Vc"] = normal(seed, stream(S_V, step), (wl.B, wl.Hkv, wl.Lcap, wl.hd), 1.0, wl.dtype)
    if wl.L is not None:
        out["lens"] = np.full(wl.B, wl.L, dtype=np.int32)
    else:
        out["lens"] = randint(seed, stream(S_LENS, step), wl.B, wl.L_range[0], wl.L_range[1])
    out["root_tok"] = randint(seed, stream(S_ROOT, step), wl.B, 0, wl.V - 1)
    if wl.rows_per_request == 1:
        out["src_row"] = np.arange(wl.B, dtype=np.int32)
    else:
        node = randint(seed, stream(S_SRC, step), wl.B, 0, wl.rows_per_request - 1)
        out["src_row"] = (np.arange(wl.B, dtype=np.int32) * wl.rows_per_request + node).astype(np.int32)
    if wl.target_head:
        out["Ht"] = normal(seed, stream(S_HT, step), (wl.B, wl.N, wl.d), 1.0, wl.dtype)
    else:
        out["logits"] = normal(seed, stream(S_LOGITS, step), (wl.B, wl.N, wl.V), 1.0, "f32")
    if wl.verify == "sampled":
        out["draft_words"] = u32(seed, stream(S_DRAFTW, step), wl.M * wl.K * wl.V).reshape(wl.M, wl.K, wl.V)
        out["u_words"] = u32(seed, stream(S_UW, step), wl.B * wl.N).reshape(wl.B, wl.N)
    if wl.verify in ("sampled", "typical"):
        out["g_words"] = u32(seed, stream(S_GW, step), wl.B * wl.V).reshape(wl.B, wl.V)
    return out


def plant(logits: np.ndarray, topo: Topology, tree_tok: np.ndarray, a: Sequence[float],
          seed: int, step: int = 0) -> np.ndarray:
    """Make the target's argmax accept depth i with probability a_i, in place.

    Per request: draw a deepest node uniformly and walk its root path. At
    depth i, with probability a_i the child's token becomes its parent row's
    unique maximum (row max + 1); otherwise every child token of that parent
    is pushed at least 1 below the best non-child logit, and the walk stops.
    Rows off the path are left as drawn. Acceptance then continues past depth
    i with probability a_i exactly, so the mean accepted length is the closed
    form of the acceptance paragraph of Medusa heads versus separate draft
    model: 1 + a1 + a1 a2 + ...
    """
    B, N, V = logits.shape
    depth = [len(p) for p in topo.paths]
    D = max(depth)
    deepest = [i for i in range(N) if depth[i] == D]
    children = [[c for c in range(N) if topo.parent[c] == p] for p in range(N)]
    u = uniform01(seed, stream(S_PLANT, step), B * (D + 1)).reshape(B, D + 1)
    for b in range(B):
        leaf = deepest[min(int(u[b, 0] * len(deepest)), len(deepest) - 1)]
        path = [leaf]
        while topo.parent[path[-1]] >= 0:
            path.append(topo.parent[path[-1]])
        path.reverse()  # root ... leaf
        for i in range(1, D + 1):
            p, c = path[i - 1], path[i]
            row = logits[b, p]
            if u[b, i] < a[i - 1]:
                row[tree_tok[b, c]] = np.float32(row.max() + np.float32(1.0))
            else:
                toks = np.array([tree_tok[b, cc] for cc in children[p]], dtype=np.int64)
                mask = np.ones(V, dtype=bool)
                mask[toks] = False
                cap = np.float32(row[mask].max() - np.float32(1.0))
                row[toks] = np.minimum(row[toks], cap)
                break
    return logits


def plant_hidden(Ht: np.ndarray, Wt: np.ndarray, topo: Topology, tree_tok: np.ndarray, a: Sequence[float],
                 seed: int, step: int = 0, alpha: float = 16.0) -> np.ndarray:
    """The acceptance plant of `plant`, made in the target's hidden states.

    Same draws and walk as `plant`. Where the walk accepts the child c of p,
    row p of Ht gets alpha * Wt[token of c] added: that token's logit grows by
    about alpha (|Wt[v]| ~ 1) while every other logit moves by ~alpha/sqrt(d),
    so the target picks it. Where the walk stops, row p gets alpha * Wt[x] for
    a drawn token x that no child of p carries. Ht and Wt are storage arrays
    (float32 or bf16 bits), Ht [B, N, d] is changed in place; the result is
    rounded back to the storage type, and both sides of a comparison read it.
    """
    from . import bf16_to_f32, f32_to_bf16

    B, N, d = Ht.shape
    V = Wt.shape[0]
    bf = Ht.dtype == np.uint16
    H = bf16_to_f32(Ht).astype(np.float64) if bf else Ht.astype(np.float64)
    W = (lambda v: bf16_to_f32(Wt[v]).astype(np.float64)) if bf else (lambda v: Wt[v].astype(np.float64))
    depth = [len(p) for p in topo.paths]
    D = max(depth)
    deepest = [i for i in range(N) if depth[i] == D]
    children = [[c for c in range(N) if topo.parent[c] == p] for p in range(N)]
    u = uniform01(seed, stream(S_PLANT, step), B * (D + 1)).reshape(B, D + 1)
    alt = randint(seed, stream(S_ALT, step), B * D * 4, 0, V - 1).reshape(B, D, 4)
    for b in range(B):
        leaf = deepest[min(int(u[b, 0] * len(deepest)), len(deepest) - 1)]
        path = [leaf]
        while topo.parent[path[-1]] >= 0:
            path.append(topo.parent[path[-1]])
        path.reverse()
        for i in range(1, D + 1):
            p, c = path[i - 1], path[i]
            if u[b, i] < a[i - 1]:
                H[b, p] += alpha * W(int(tree_tok[b, c]))
            else:
                taken = {int(tree_tok[b, cc]) for cc in children[p]}
                x = next((int(v) for v in alt[b, i - 1] if int(v) not in taken), None)
                if x is None:  # four draws all hit a child token: take the lowest free index
                    x = next(v for v in range(V) if v not in taken)
                H[b, p] += alpha * W(x)
                break
    Ht[...] = f32_to_bf16(H.astype(np.float32)) if bf else H.astype(Ht.dtype)
    return Ht
