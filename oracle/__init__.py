"""CPU oracle for the Medusa tree-decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg import this package. The GPU library (``medusa_draft_heads_amd``) never
imports it and shares no code with it; the two meet only through the seeded
inputs of ``synth``.

The arithmetic lives in ``oracle.c`` (plain loops, double precision). This
module marshals numpy arrays and orchestrates the steps in the order the
pages give them:

* heads -- Medusa heads versus separate draft model, "What each one is":
  every head is a residual block on the target's last hidden state followed
  by its own vocabulary projection;
* per-head top-k and the tree of combinations -- same page, "Trees";
* tree-masked attention over the KV cache -- same page, "Trees";
* greedy acceptance and the cache entries of the accepted branch -- same
  page, "Trees" and "Acceptance";
* Hydra heads -- the Hydra summary and abstract: each head also sees the
  token speculated before it;
* sampled decoding -- same page, "Training": rejection sampling with the
  heads' probabilities (exact) and typical acceptance (not exact); the
  readings for a tree are stated at that section below.

bf16 arrays are numpy uint16 bit patterns; float32 arrays are float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        i, i64, d, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        sig = {
            "orc_set_threads": ([i], None),
            "orc_get_threads": ([], i),
            "orc_to_double": ([i, i64, vp, vp], None),
            "orc_head_weight_elems": ([i, i, i], i64),
            "orc_residual": ([i, i, i, i, vp, vp, vp, vp, vp], None),
            "orc_vocab_topk": ([i, i, i, i, vp, vp, i, vp, vp, vp, vp], None),
            "orc_tree_tokens_medusa": ([i, vp, vp, i, i, i, vp, vp, vp, vp, vp, vp], None),
            "orc_tree_attention": ([i, i, i, vp, i, i, i, i, vp, vp, vp, vp, d, vp], None),
            "orc_argmax": ([i64, i, vp, vp], None),
            "orc_accept": ([i, vp, i, i, vp, vp, vp, vp, vp, vp, vp], None),
            "orc_compact": ([i, i, i, i, i, vp, vp, vp, vp, vp, i], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError("storage dtype must be float32 or uint16 (bf16 bits), got %s" % a.dtype)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def threads() -> int:
    return int(lib().orc_get_threads())


def to_double(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, dtype=np.float64)
    lib().orc_to_double(_dt(a), a.size, _p(a), _p(out))
    return out


def head_weight_elems(din: int, d: int, V: int) -> int:
    return int(lib().orc_head_weight_elems(din, d, V))


# ------------------------------------------------------------------ heads

def residual(W_k: np.ndarray, b_k: Optional[np.ndarray], x: np.ndarray, base: np.ndarray) -> np.ndarray:
    """hres = base + SiLU(W_k x + b_k) for every row of x (double in, double out)."""
    d, din = W_k.shape
    x = np.ascontiguousarray(x, dtype=np.float64)
    base = np.ascontiguousarray(base, dtype=np.float64)
    M = x.shape[0]
    assert x.shape == (M, din) and base.shape == (M, d)
    out = np.empty((M, d), dtype=np.float64)
    if b_k is not None:
        assert b_k.dtype == W_k.dtype
    lib().orc_residual(_dt(W_k), M, din, d, _p(x), _p(base), _p(np.ascontiguousarray(W_k)),
                       _p(None if b_k is None else np.ascontiguousarray(b_k)), _p(out))
    return out


def vocab_topk(U_k: np.ndarray, hres: np.ndarray, k: int, want_logits: bool = False):
    """Top-k of U_k hres per row, sorted by (value desc, index asc), and its margin."""
    V, d = U_k.shape
    hres = np.ascontiguousarray(hres, dtype=np.float64)
    M = hres.shape[0]
    idx = np.empty((M, k), dtype=np.int32)
    val = np.empty((M, k), dtype=np.float64)
    margin = np.empty(M, dtype=np.float64)
    logits = np.empty((M, V), dtype=np.float64) if want_logits else None
    lib().orc_vocab_topk(_dt(U_k), M, d, V, _p(hres), _p(np.ascontiguousarray(U_k)), k,
                         _p(idx), _p(val), _p(margin), _p(logits))
    return idx, val, margin, logits


def target_argmax(H, Wt):
    """The target's greedy choice per row of its final hidden states H [R, d]
    through its LM head Wt [V, d] ("Medusa heads versus separate draft model",
    Trees: one verification pass over the tree): the first index of the
    largest logit, with that logit and the gap to the runner-up (the top-1
    list and its margin)."""
    i_, v_, m_, _ = vocab_topk(Wt, to_double(H), 1)
    return i_[:, 0], v_[:, 0], m_


def heads_medusa(W, b, U, h, topk: Sequence[int], rows: Optional[Sequence[int]] = None,
                 want_logits: bool = False) -> Dict[str, np.ndarray]:
    """All K Medusa heads on hidden-state rows h [M, d].

    U is [K, V, d], or [V, d] for one projection shared by every head ("Medusa
    heads versus separate draft model", What interviewers probe next).
    Returns hres [K, R, d], idx [R, K, kmax] (-1 padded), val [R, K, kmax]
    (-inf padded), margin [R, K], for the R selected rows (all by default),
    and with want_logits the full logits [R, K, V].
    """
    K = W.shape[0]
    hd = to_double(h)
    if rows is not None:
        hd = hd[np.asarray(rows)]
    R, d = hd.shape
    kmax = max(topk)
    hres = np.empty((K, R, d), dtype=np.float64)
    idx = np.full((R, K, kmax), -1, dtype=np.int32)
    val = np.full((R, K, kmax), -np.inf, dtype=np.float64)
    margin = np.empty((R, K), dtype=np.float64)
    logits = np.empty((R, K, U.shape[-2]), dtype=np.float64) if want_logits else None
    for k in range(K):
        hres[k] = residual(W[k], b[k], hd, hd)
        i_, v_, m_, lg = vocab_topk(U if U.ndim == 2 else U[k], hres[k], topk[k], want_logits=want_logits)
        idx[:, k, : topk[k]] = i_
        val[:, k, : topk[k]] = v_
        margin[:, k] = m_
        if want_logits:
            logits[:, k] = lg
    out = {"hres": hres, "idx": idx, "val": val, "margin": margin}
    if want_logits:
        out["logits"] = logits
    return out


def _depths(parent: Sequence[int]):
    dep = []
    for n in range(len(parent)):
        d, c = 0, n
        while parent[c] >= 0:
            c = parent[c]
            d += 1
        dep.append(d)
    return dep


def hydra_rows(parent: Sequence[int], level: int):
    """Parents whose children sit at depth `level`, in node order."""
    dep = _depths(parent)
    return [p for p in range(len(parent)) if dep[p] == level - 1 and any(parent[c] == p for c in range(len(parent)))]


def hydra_level(W, b, U, E, h, topo_parent, topo_rank, topk: Sequence[int], level: int, tree_tok,
                requests: Optional[Sequence[int]] = None, want_logits: bool = False) -> Dict[str, object]:
    """Hydra's level `level` (the Hydra summary and abstract), given the tree's
    tokens at depths below it (tree_tok [B, N]; the root at node 0).

    One row per (request, parent at depth level - 1 with children), in node
    order: x = [h_b ; E[token of the parent]] (a token outside [0, V) embeds as
    zeros), hres = h_b + SiLU(W_i x + b_i), then head i's projection and
    top-k_i. Returns the rows, hres, idx, val, margin (and the logits), and the
    tokens of the depth-`level` nodes: entry rank(n) of the node's own
    parent's list.
    """
    i = level
    N = len(topo_parent)
    dep = _depths(topo_parent)
    B = h.shape[0]
    reqs = list(range(B)) if requests is None else list(requests)
    hd = to_double(h)
    V = E.shape[0]
    Ed_cache: Dict[int, np.ndarray] = {}

    def emb(tok: int) -> np.ndarray:
        # a token outside [0, V) names no row of E: it embeds as zeros
        if tok not in Ed_cache:
            if 0 <= tok < V:
                Ed_cache[tok] = to_double(np.ascontiguousarray(E[tok]))
            else:
                Ed_cache[tok] = np.zeros(E.shape[1], dtype=np.float64)
        return Ed_cache[tok]

    parents = hydra_rows(topo_parent, i)
    rows = [(b_, p) for b_ in reqs for p in parents]
    if not rows:
        return {"rows": [], "tok": {}}
    x = np.stack([np.concatenate([hd[b_], emb(int(tree_tok[b_, p]))]) for (b_, p) in rows])
    base = np.stack([hd[b_] for (b_, _) in rows])
    hres = residual(W[i - 1], b[i - 1], x, base)
    idx, val, margin, lg = vocab_topk(U[i - 1], hres, topk[i - 1], want_logits=want_logits)
    row_of = {rp: r for r, rp in enumerate(rows)}
    tok = {(b_, n): int(idx[row_of[(b_, topo_parent[n])], topo_rank[n]])
           for b_ in reqs for n in range(N) if dep[n] == i}
    return {"rows": rows, "hres": hres, "idx": idx, "val": val, "margin": margin, "logits": lg, "tok": tok}


def hydra_expand(W, b, U, E, h, topo_parent, topo_rank, topk: Sequence[int], root_tok, lens,
                 requests: Optional[Sequence[int]] = None, want_logits: bool = False) -> Dict[str, object]:
    """Hydra heads, level by level (the Hydra summary and abstract): level i
    runs head i on one row per (request, parent at depth i - 1 with children)
    and each depth-i node takes entry rank(n) of its own parent's list
    (hydra_level). Returns the tree tokens, positions and every level's
    (rows, hres, idx, val, margin).
    """
    K = W.shape[0]
    N = len(topo_parent)
    dep = _depths(topo_parent)
    B = h.shape[0]
    reqs = list(range(B)) if requests is None else list(requests)
    tok = np.full((B, N), -1, dtype=np.int32)
    pos = np.zeros((B, N), dtype=np.int32)
    for b_ in reqs:
        tok[b_, 0] = root_tok[b_]
        for n in range(N):
            pos[b_, n] = lens[b_] + dep[n]
    levels = []
    for i in range(1, K + 1):
        lvl = hydra_level(W, b, U, E, h, topo_parent, topo_rank, topk, i, tok, requests=reqs,
                          want_logits=want_logits)
        if not lvl["rows"]:
            break
        for (b_, n), t in lvl.pop("tok").items():
            tok[b_, n] = t
        levels.append(lvl)
    return {"tree_tok": tok, "tree_pos": pos, "levels": levels}


# ------------------------------------------------------------------ tree

def tree_tokens_medusa(parent, rank, topk_idx: np.ndarray, src_row, root_tok, lens):
    M, K, kmax = topk_idx.shape
    N = len(parent)
    B = len(root_tok)
    par = np.asarray(parent, dtype=np.int8)
    rk = np.asarray(rank, dtype=np.int8)
    tok = np.empty((B, N), dtype=np.int32)
    pos = np.empty((B, N), dtype=np.int32)
    lib().orc_tree_tokens_medusa(N, _p(par), _p(rk), B, K, kmax, _p(np.ascontiguousarray(topk_idx, dtype=np.int32)),
                                 _p(np.ascontiguousarray(src_row, dtype=np.int32)),
                                 _p(np.ascontiguousarray(root_tok, dtype=np.int32)),
                                 _p(np.ascontiguousarray(lens, dtype=np.int32)), _p(tok), _p(pos))
    return tok, pos


def tree_attention(parent, q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, lens, scale: Optional[float] = None):
    B, N, Hq, hd = q.shape
    _, Hkv, Lcap, _ = Kc.shape
    assert len(parent) == N and Kc.shape == Vc.shape and Hq % Hkv == 0
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    out = np.empty((B, N, Hq, hd), dtype=np.float64)
    par = np.asarray(parent, dtype=np.int8)
    lib().orc_tree_attention(_dt(q), B, N, _p(par), Hq, Hkv, hd, Lcap, _p(np.ascontiguousarray(q)),
                             _p(np.ascontiguousarray(Kc)), _p(np.ascontiguousarray(Vc)),
                             _p(np.ascontiguousarray(lens, dtype=np.int32)), float(scale), _p(out))
    return out


# --------------------------------------------------------- verify / accept

def argmax(logits: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(logits, dtype=np.float32)
    V = x.shape[-1]
    R = x.size // V
    out = np.empty(R, dtype=np.int32)
    lib().orc_argmax(R, V, _p(x), _p(out))
    return out.reshape(x.shape[:-1])


def accept(parent, K: int, tree_tok: np.ndarray, tstar: np.ndarray, lens):
    B, N = tree_tok.shape
    par = np.asarray(parent, dtype=np.int8)
    acc = np.empty(B, dtype=np.int32)
    path = np.empty((B, K + 1), dtype=np.int32)
    nxt = np.empty(B, dtype=np.int32)
    src = np.empty((B, K + 1), dtype=np.int32)
    lib().orc_accept(N, _p(par), B, K, _p(np.ascontiguousarray(tree_tok, dtype=np.int32)),
                     _p(np.ascontiguousarray(tstar, dtype=np.int32)),
                     _p(np.ascontiguousarray(lens, dtype=np.int32)), _p(acc), _p(path), _p(nxt), _p(src))
    return {"accept_len": acc, "path": path, "next_tok": nxt, "compact_src": src}


def compact(Kc: np.ndarray, Vc: np.ndarray, lens, accept_len, path, K: int):
    """In place on copies: returns (Kc', Vc', lens')."""
    Kc = np.ascontiguousarray(Kc).copy()
    Vc = np.ascontiguousarray(Vc).copy()
    B, Hkv, Lcap, hd = Kc.shape
    ln = np.ascontiguousarray(lens, dtype=np.int32).copy()
    lib().orc_compact(_dt(Kc), B, Hkv, hd, Lcap, _p(Kc), _p(Vc), _p(ln),
                      _p(np.ascontiguousarray(accept_len, dtype=np.int32)),
                      _p(np.ascontiguousarray(path, dtype=np.int32)), K)
    return Kc, Vc, ln


def step_medusa(wl, wts: Dict[str, np.ndarray], inp: Dict[str, np.ndarray], topo, logits: np.ndarray):
    """One whole decode step on the CPU: heads, tree, attention, verification, accept, compaction."""
    K = wl.K
    heads = heads_medusa(wts["W"], wts["b"], wts["U"], inp["h"], wl.topk,
                         rows=sorted(set(int(r) for r in inp["src_row"])))
    # heads ran on the distinct source rows only; map them back to row ids
    rows = sorted(set(int(r) for r in inp["src_row"]))
    full_idx = np.full((wl.M, K, wl.kmax), -1, dtype=np.int32)
    for j, r in enumerate(rows):
        full_idx[r] = heads["idx"][j]
    tok, pos = tree_tokens_medusa(topo.parent, topo.rank, full_idx, inp["src_row"], inp["root_tok"], inp["lens"])
    out = tree_attention(topo.parent, inp["q"], inp["Kc"], inp["Vc"], inp["lens"])
    tstar = argmax(logits)
    acc = accept(topo.parent, K, tok, tstar, inp["lens"])
    Kc2, Vc2, lens2 = compact(inp["Kc"], inp["Vc"], inp["lens"], acc["accept_len"], acc["path"], K)
    return {"heads": heads, "tree_tok": tok, "tree_pos": pos, "attn": out, "tstar": tstar, **acc,
            "Kc": Kc2, "Vc": Vc2, "lens": lens2}


# ------------------------------------------------ sampled decoding
#
# "Medusa heads versus separate draft model", Training: for sampled decoding
# at a temperature, an exact match of the target's distribution needs
# standard rejection sampling with the heads' probabilities; Medusa's
# "typical acceptance" takes more drafts but gives that up. The pages do not
# spell out either procedure on a tree; the readings taken here:
#
# * a head's draft distribution is q = softmax(logits / T), the target's at
#   node n is p_n = softmax(target_logits[n] / T);
# * a head's draft tokens are a sample of k distinct tokens from q in draw
#   order (Gumbel-top-k: the k largest of logits / T + Gumbel noise);
# * verification walks down from the root; at a node, its children are tried
#   in rank order with the rejection rule for candidates drawn without
#   replacement: accept child x with probability min(1, p(x) / q(x)); on
#   rejection p <- normalise(max(0, p - q)) and x leaves q (q renormalised).
#   An accepted child becomes the node; when every child is rejected, or the
#   node is a leaf, the step's last token is drawn from the current p; a
#   tree token outside [0, V) is never accepted and changes nothing;
# * typical acceptance: a node matches when its parent's p gives its token
#   more than min(eps, delta * exp(-entropy(p))); the deepest node whose
#   whole root path matches ends the step, and the last token is drawn from
#   that node's p.
#
# Random numbers come in as 32-bit words: uniforms u = (w / 2^9 + 1/2) 2^-23
# in (0, 1) and Gumbel noise -log(-log u).


def unit_from_words(w) -> np.ndarray:
    """Uniforms in the open interval (0, 1): the top 23 bits of each word plus one half, times 2^-23."""
    w = np.asarray(w, dtype=np.uint32)
    return ((w >> np.uint32(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel_from_words(w) -> np.ndarray:
    """Standard Gumbel noise -log(-log u) of the uniforms above."""
    return -np.log(-np.log(unit_from_words(w)))


def softmax_t(x, T: float) -> np.ndarray:
    z = np.asarray(x, dtype=np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def logsumexp_t(x, T: float) -> float:
    z = np.asarray(x, dtype=np.float64) / T
    m = z.max()
    return float(m + np.log(np.exp(z - m).sum()))


def _order_desc(s: np.ndarray) -> np.ndarray:
    """Indices by (value desc, index asc)."""
    return np.lexsort((np.arange(s.size), -s))


def draft_sample(logits: np.ndarray, words: np.ndarray, topk: Sequence[int], T: float) -> Dict[str, np.ndarray]:
    """Per (row, head): k_head distinct tokens drawn without replacement from
    softmax(logits / T), in draw order (the k largest of logits / T + Gumbel
    noise), and log sum exp(logits / T).

    logits [R, K, V], words [R, K, V] uint32. Returns tok [R, K, kmax] (-1
    padded), score [R, K, kmax] (the perturbed values), lse [R, K] and
    margin [R, K]: the smallest gap among the k + 1 best perturbed values.
    """
    R, K, V = logits.shape
    kmax = max(topk)
    tok = np.full((R, K, kmax), -1, dtype=np.int32)
    score = np.full((R, K, kmax), -np.inf)
    lse = np.empty((R, K))
    margin = np.empty((R, K))
    for r in range(R):
        for k in range(K):
            s = np.asarray(logits[r, k], dtype=np.float64) / T + gumbel_from_words(words[r, k])
            o = _order_desc(s)
            kk = topk[k]
            tok[r, k, :kk] = o[:kk]
            score[r, k, :kk] = s[o[:kk]]
            top = s[o[: min(kk + 1, V)]]
            margin[r, k] = np.min(top[:-1] - top[1:]) if top.size > 1 else np.inf
            lse[r, k] = logsumexp_t(logits[r, k], T)
    return {"tok": tok, "score": score, "lse": lse, "margin": margin}


def _children(parent: Sequence[int]):
    ch = [[] for _ in parent]
    for n in range(1, len(parent)):
        ch[parent[n]].append(n)  # breadth-first numbering: siblings in rank order
    return ch


def _gumbel_max(p: np.ndarray, gw: np.ndarray):
    """A draw from p (Gumbel-max over log p) and the gap between the two best perturbed values."""
    with np.errstate(divide="ignore"):
        s = np.log(p) + gumbel_from_words(gw)
    o = _order_desc(s)
    gap = s[o[0]] - s[o[1]] if s.size > 1 else np.inf
    return int(o[0]), float(gap)


def verify_sampled(parent: Sequence[int], tree_tok: np.ndarray, target_logits: np.ndarray, head_logits: np.ndarray,
                   T: float, u_words: np.ndarray, g_words: np.ndarray) -> Dict[str, np.ndarray]:
    """Rejection-sampling verification of the tree (readings above).

    tree_tok [B, N]; target_logits [B, N, V] (the target at every node);
    head_logits [B, K, V] (the heads that drafted request b's tree: head i
    supplies the depth-(i+1) tokens); u_words [B, N] (node n's acceptance
    test); g_words [B, V] (the final draw). Returns chosen [B, N] (the token
    emitted after each node the walk passed through, -1 elsewhere; node a's
    entry is the step's last token) and margin [B]: the smallest distance
    between a test's uniform and its acceptance probability, and the gap of
    the final draw's two best perturbed values.
    """
    B, N = tree_tok.shape
    dep = _depths(parent)
    ch = _children(parent)
    chosen = np.full((B, N), -1, dtype=np.int32)
    margin = np.full(B, np.inf)
    for b_ in range(B):
        node = 0
        while True:
            p = softmax_t(target_logits[b_, node], T)
            kids = ch[node]
            q = softmax_t(head_logits[b_, dep[node]], T) if kids else None
            nxt = None
            for c in kids:
                x = int(tree_tok[b_, c])
                if not 0 <= x < p.size:
                    continue  # not a token: never accepted, changes nothing
                u = float(unit_from_words(u_words[b_, c]))
                a = min(1.0, p[x] / q[x]) if q[x] > 0.0 else 1.0
                margin[b_] = min(margin[b_], abs(u - a))
                if u < a:
                    nxt = c
                    break
                r = np.maximum(p - q, 0.0)
                p = r / r.sum()
                q = q.copy()
                q[x] = 0.0
                q = q / q.sum()
            if nxt is not None:
                chosen[b_, node] = tree_tok[b_, nxt]
                node = nxt
                continue
            y, gap = _gumbel_max(p, g_words[b_])
            chosen[b_, node] = y
            margin[b_] = min(margin[b_], gap)
            break
    return {"chosen": chosen, "margin": margin}


def typical_accept(parent: Sequence[int], tree_tok: np.ndarray, target_logits: np.ndarray, T: float, eps: float,
                   delta: float, g_words: np.ndarray) -> Dict[str, np.ndarray]:
    """Typical acceptance (reading above). Returns chosen [B, N] as
    verify_sampled does, match [B, N] (bool), the threshold and p(token) of
    every non-root node, and margin [B]: the smallest |p(token) / threshold
    - 1| and the final draw's gap."""
    B, N = tree_tok.shape
    dep = _depths(parent)
    chosen = np.full((B, N), -1, dtype=np.int32)
    match = np.zeros((B, N), dtype=bool)
    thr = np.full((B, N), np.nan)
    ptok = np.full((B, N), np.nan)
    margin = np.full(B, np.inf)
    for b_ in range(B):
        P = {}
        for n in range(1, N):
            a = parent[n]
            if a not in P:
                p = softmax_t(target_logits[b_, a], T)
                with np.errstate(divide="ignore", invalid="ignore"):
                    H = -np.sum(np.where(p > 0.0, p * np.log(p), 0.0))
                P[a] = (p, min(eps, delta * np.exp(-H)))
            p, t = P[a]
            thr[b_, n] = t
            x = int(tree_tok[b_, n])
            ptok[b_, n] = p[x] if 0 <= x < p.size else 0.0  # not a token: probability 0
            match[b_, n] = ptok[b_, n] > t
            if t > 0.0:
                margin[b_] = min(margin[b_], abs(ptok[b_, n] / t - 1.0))
        # deepest node whose whole root path matches; lowest index among equals
        best = 0
        for n in range(1, N):
            ok, c = True, n
            while c > 0:
                ok &= bool(match[b_, c])
                c = parent[c]
            if ok and dep[n] > dep[best]:
                best = n
        c = best
        while c > 0:
            chosen[b_, parent[c]] = tree_tok[b_, c]
            c = parent[c]
        y, gap = _gumbel_max(softmax_t(target_logits[b_, best], T), g_words[b_])
        chosen[b_, best] = y
        margin[b_] = min(margin[b_], gap)
    return {"chosen": chosen, "match": match, "thr": thr, "ptok": ptok, "margin": margin}
