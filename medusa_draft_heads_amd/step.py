"""One Medusa (or Hydra) tree-decode step through libmedusa.

MedusaStep owns the outputs and workspaces of a fixed configuration and issues
the four library calls in the order the step needs them: heads -> tree ->
tree attention -> accept. Hydra runs its heads level by level, each level's
tree tokens feeding the next level's embedding lookup. With target_head the
verification starts from the target's final hidden states: its LM head with
a fused argmax gives the target's choice per node, then acceptance. Sampled
decoding ("sampled") draws the drafts from the heads' full logits and verifies
by rejection sampling; "typical" keeps the top-k drafts and verifies by
typical acceptance. Buffers are allocated once, so a step allocates nothing
and issues no host synchronisation.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import torch

from . import _lib as L


@dataclass
class StepConfig:
    kind: int  # L.MD_HEADS_MEDUSA, L.MD_HEADS_HYDRA or L.MD_HEADS_MEDUSA_SHARED (U is [V][d])
    dtype: torch.dtype  # storage type of activations, weights and cache
    B: int  # requests
    M: int  # rows of h through the heads (Medusa: B or B*N; Hydra: B)
    d: int
    V: int
    K: int
    k_per_head: Sequence[int]
    parent: Sequence[int]
    rank: Sequence[int]
    Hq: int
    Hkv: int
    hd: int
    Lcap: int
    max_len: int
    target_head: bool = False  # verify from hidden states Ht [B, N, d] through the LM head Wt [V, d]
    verify: str = "greedy"  # "greedy", "sampled" (Medusa kinds, M == B) or "typical"
    temperature: float = 1.0
    eps: float = 0.09
    delta: float = 0.3


class MedusaStep:
    def __init__(self, cfg: StepConfig, device: str = "cuda"):
        self.cfg = cfg
        self.dev = torch.device(device)
        self.dt = L.MD_F32 if cfg.dtype == torch.float32 else L.MD_BF16
        self.tree = L.make_tree(cfg.parent, cfg.rank)
        rc = L.md_tree_validate(self.tree, cfg.K, cfg.k_per_head)
        if rc != L.MD_OK:
            raise L.MedusaError(rc, L.md_last_error())
        self.N = len(cfg.parent)
        self.kmax = max(cfg.k_per_head)
        i32 = dict(dtype=torch.int32, device=self.dev)
        B, N, K = cfg.B, self.N, cfg.K
        if cfg.kind != L.MD_HEADS_HYDRA:
            self.topk_idx = torch.empty(cfg.M, K, self.kmax, **i32)
            self.topk_val = torch.empty(cfg.M, K, self.kmax, dtype=torch.float32, device=self.dev)
        else:
            # one list per (request, parent) row of the widest level
            self.topk_idx = torch.empty(B * N, 1, self.kmax, **i32)
            self.topk_val = torch.empty(B * N, 1, self.kmax, dtype=torch.float32, device=self.dev)
        self.tree_tok = torch.empty(B, N, **i32)
        self.tree_pos = torch.empty(B, N, **i32)
        self.attn_out = torch.empty(B, N, cfg.Hq, cfg.hd, dtype=cfg.dtype, device=self.dev)
        self.accept_len = torch.empty(B, **i32)
        self.path = torch.empty(B, K + 1, **i32)
        self.next_tok = torch.empty(B, **i32)
        self.compact_src = torch.empty(B, K + 1, **i32)
        u8 = dict(dtype=torch.uint8, device=self.dev)
        self.ws_heads = torch.empty(max(1, L.md_heads_workspace_bytes(cfg.kind, self.dt, cfg.M, cfg.d, cfg.V, K,
                                                                       self.kmax)), **u8)
        self.ws_attn = torch.empty(max(1, L.md_attention_workspace_bytes(self.dt, B, N, cfg.Hq, cfg.Hkv, cfg.hd,
                                                                          cfg.max_len)), **u8)
        self.ws_acc = torch.empty(max(1, L.md_accept_workspace_bytes(B, N, cfg.V)), **u8)
        if cfg.target_head:
            self.target_tok = torch.empty(B, N, **i32)
            self.target_val = torch.empty(B, N, dtype=torch.float32, device=self.dev)
            self.ws_target = torch.empty(max(1, L.md_target_argmax_workspace_bytes(self.dt, B * N, cfg.d, cfg.V)),
                                         **u8)
        if cfg.verify == "sampled":
            if cfg.kind == L.MD_HEADS_HYDRA or cfg.M != B or cfg.target_head:
                raise ValueError("sampled verification takes Medusa heads on one row per request")
            f32 = dict(dtype=torch.float32, device=self.dev)
            self.head_logits = torch.empty(B, K, cfg.V, **f32)
            self.head_lse = torch.empty(B, K, **f32)
            self.ws_logits = torch.empty(max(1, L.md_heads_logits_workspace_bytes(cfg.kind, B, cfg.d, K)), **u8)
            self.ws_draft = torch.empty(max(1, L.md_draft_sample_workspace_bytes(B, K, cfg.V, self.kmax)), **u8)
            self.ws_vs = torch.empty(max(1, L.md_verify_sampled_workspace_bytes(B, N)), **u8)
        elif cfg.verify == "typical":
            self.ws_typ = torch.empty(max(1, L.md_accept_typical_workspace_bytes(B, N)), **u8)
        elif cfg.verify != "greedy":
            raise ValueError("verify = %r" % cfg.verify)
        self.scale = 1.0 / float(cfg.hd) ** 0.5
        self.h_res = None

    # -- the four calls -------------------------------------------------------
    def heads(self, h, W, b, U, E=None, root_tok=None, level: int = 0, h_res=None, U_op=None, U_norms=None,
              W_op=None) -> None:
        c = self.cfg
        L.md_medusa_heads(c.kind, self.dt, c.M, c.d, c.V, c.K, c.k_per_head, level, self.tree, h, W, b, U, E,
                          root_tok, self.tree_tok, self.topk_idx, self.topk_val, h_res, self.ws_heads, U_op=U_op,
                          U_norms=U_norms, W_op=W_op)

    def build(self, src_row, root_tok, lens, level: int = 0) -> None:
        c = self.cfg
        L.md_tree_build(self.tree, c.kind, c.B, c.M, c.K, self.kmax, level, self.topk_idx, src_row, root_tok, lens,
                        self.tree_tok, self.tree_pos)

    def attention(self, q, Kc, Vc, lens) -> None:
        c = self.cfg
        L.md_tree_attention(self.tree, self.dt, c.B, c.Hq, c.Hkv, c.hd, c.Lcap, c.max_len, q, Kc, Vc, lens,
                            self.scale, self.attn_out, self.ws_attn)

    def accept(self, logits, Kc, Vc, lens) -> None:
        c = self.cfg
        L.md_tree_accept(self.tree, self.dt, c.B, c.K, c.V, c.Hkv, c.hd, c.Lcap, logits, self.tree_tok, Kc, Vc, lens,
                         self.accept_len, self.path, self.next_tok, self.compact_src, self.ws_acc)

    def verify(self, Ht, Wt, Wt_op=None) -> None:
        """The target's choice at every node: LM head + fused argmax over Ht [B, N, d]."""
        c = self.cfg
        L.md_target_argmax(self.dt, c.B * self.N, c.d, c.V, Ht, Wt, self.target_tok, self.target_val, self.ws_target,
                           Wt_op=Wt_op)

    def tile_norm_weights(self, w: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
        """The tile norms of the vocabulary matrices (U_norms), made once when the weights load; bf16 only.
        run() passes them on when w holds them (the many-row certified pass reads them)."""
        if self.dt != L.MD_BF16:
            raise ValueError("tile norms exist for bf16 weights only")
        return {"U_norms": L.vocab_tile_norms(w["U"])}

    def operand_order_weights(self, w: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
        """Operand-order copies of the vocabulary matrices (U_op, and Wt_op with target_head) and of the
        residual matrices (W_op), made once
        when the weights load; bf16 only. run() passes them on when w holds them."""
        if self.dt != L.MD_BF16:
            raise ValueError("operand-order copies exist for bf16 weights only")
        out = {"U_op": L.operand_order(w["U"])}
        # W's copy only where a few-row matrix-core residual reads it (Hydra's levels, 2 to 77 Medusa
        # rows); one row runs the fused or GEMV residual on W itself
        if self.cfg.kind == L.MD_HEADS_HYDRA or 1 < self.cfg.M < 78:
            out["W_op"] = L.operand_order(w["W"])
        if self.cfg.target_head:
            out["Wt_op"] = L.operand_order(w["Wt"])
        return out

    def accept_tokens(self, Kc, Vc, lens) -> None:
        c = self.cfg
        L.md_tree_accept_tokens(self.tree, self.dt, c.B, c.K, c.Hkv, c.hd, c.Lcap, self.target_tok, self.tree_tok, Kc,
                                Vc, lens, self.accept_len, self.path, self.next_tok, self.compact_src)

    # -- sampled decoding ---------------------------------------------------------
    def heads_logits(self, h, W, b, U) -> None:
        c = self.cfg
        L.md_medusa_heads_logits(c.kind, self.dt, c.M, c.d, c.V, c.K, h, W, b, U, self.head_logits, None,
                                 self.ws_logits)

    def draft(self, words) -> None:
        c = self.cfg
        L.md_draft_sample(c.M, c.K, c.V, c.k_per_head, c.temperature, self.head_logits, words, self.topk_idx,
                          self.head_lse, self.ws_draft)

    def verify_sampled(self, logits, u_words, g_words, Kc, Vc, lens) -> None:
        c = self.cfg
        L.md_tree_verify_sampled(self.tree, self.dt, c.B, c.K, c.V, c.Hkv, c.hd, c.Lcap, c.temperature, logits,
                                 self.head_logits, self.head_lse, self.tree_tok, u_words, g_words, Kc, Vc, lens,
                                 self.accept_len, self.path, self.next_tok, self.compact_src, self.ws_vs)

    def accept_typical(self, logits, g_words, Kc, Vc, lens) -> None:
        c = self.cfg
        L.md_tree_accept_typical(self.tree, self.dt, c.B, c.K, c.V, c.Hkv, c.hd, c.Lcap, c.temperature, c.eps, c.delta,
                                 logits, self.tree_tok, g_words, Kc, Vc, lens, self.accept_len, self.path,
                                 self.next_tok, self.compact_src, self.ws_typ)

    # -- a whole step -----------------------------------------------------------
    def run(self, w: Dict[str, torch.Tensor], x: Dict[str, torch.Tensor]) -> None:
        """w: W, b, U (E for Hydra, Wt with target_head; optionally U_op and Wt_op from
        operand_order_weights); x: h, q, Kc, Vc, lens, root_tok, src_row, and logits (or Ht with
        target_head); sampled decoding adds draft_words, u_words and g_words, typical acceptance g_words."""
        c = self.cfg
        if c.verify == "sampled":
            self.heads_logits(x["h"], w["W"], w["b"], w["U"])
            self.draft(x["draft_words"])
            self.build(x["src_row"], x["root_tok"], x["lens"])
            self.attention(x["q"], x["Kc"], x["Vc"], x["lens"])
            self.verify_sampled(x["logits"], x["u_words"], x["g_words"], x["Kc"], x["Vc"], x["lens"])
            return
        if c.kind != L.MD_HEADS_HYDRA:
            self.heads(x["h"], w["W"], w["b"], w["U"], U_op=w.get("U_op"), U_norms=w.get("U_norms"), W_op=w.get("W_op"))
            self.build(x["src_row"], x["root_tok"], x["lens"])
        else:
            depth = max(self._depths())
            for level in range(1, depth + 1):
                self.heads(x["h"], w["W"], w["b"], w["U"], E=w["E"], root_tok=x["root_tok"], level=level,
                           U_op=w.get("U_op"), U_norms=w.get("U_norms"), W_op=w.get("W_op"))
                self.build(None, x["root_tok"], x["lens"], level=level)
        self.attention(x["q"], x["Kc"], x["Vc"], x["lens"])
        if c.target_head:
            self.verify(x["Ht"], w["Wt"], w.get("Wt_op"))
            self.accept_tokens(x["Kc"], x["Vc"], x["lens"])
        elif c.verify == "typical":
            self.accept_typical(x["logits"], x["g_words"], x["Kc"], x["Vc"], x["lens"])
        else:
            self.accept(x["logits"], x["Kc"], x["Vc"], x["lens"])

    def _depths(self):
        dep = []
        for n, p in enumerate(self.cfg.parent):
            dep.append(0 if p < 0 else dep[p] + 1)
        return dep
