"""ctypes binding of libmedusa (include/medusa.h): argument marshalling only.

Every function carries the C name and forwards to the C call; tensors are
passed as raw device pointers and the stream as torch's current HIP stream.
A non-zero status raises MedusaError with the library's message. There is no
fallback: without the built library every call fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmedusa.so")

MD_OK, MD_EINVAL, MD_EUNSUPPORTED, MD_ERANGE, MD_EWORKSPACE, MD_EHIP = 0, -1, -2, -3, -4, -5
MD_F32, MD_BF16 = 0, 1
MD_HEADS_MEDUSA, MD_HEADS_HYDRA, MD_HEADS_MEDUSA_SHARED = 0, 1, 2
MD_MAX_NODES, MD_MAX_HEADS, MD_MAX_TOPK = 64, 8, 16

EXPORTS = (
    "md_tree_validate", "md_heads_weight_bytes", "md_heads_workspace_bytes", "md_medusa_heads", "md_tree_build",
    "md_attention_workspace_bytes", "md_tree_attention", "md_accept_workspace_bytes", "md_tree_accept",
    "md_set_vocab_timing_events", "md_last_error", "md_hbm_read_probe", "md_hbm_read_probe_blocks",
    "md_target_argmax_workspace_bytes", "md_target_argmax", "md_tree_accept_tokens",
    "md_heads_logits_workspace_bytes", "md_medusa_heads_logits", "md_draft_sample_workspace_bytes", "md_draft_sample",
    "md_verify_sampled_workspace_bytes", "md_tree_verify_sampled", "md_accept_typical_workspace_bytes",
    "md_tree_accept_typical", "md_operand_order_bytes", "md_operand_order", "md_certified_rounding_allowance",
    "md_vocab_tile_norms_bytes", "md_vocab_tile_norms",
    "md_tree_attention_noalloc", "md_tree_attention_noalloc_max_bytes", "md_heads_fused", "md_set_wait_limits",
)


class MedusaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("libmedusa status %d: %s" % (status, msg))
        self.status = status


class md_tree(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("parent", ctypes.c_int8 * MD_MAX_NODES), ("rank", ctypes.c_int8 * MD_MAX_NODES)]


def make_tree(parent: Sequence[int], rank: Sequence[int]) -> md_tree:
    t = md_tree()
    t.n = len(parent)
    for i, (p, r) in enumerate(zip(parent, rank)):
        t.parent[i] = p
        t.rank[i] = r
    return t


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmedusa.so is not built (run: python -m medusa_draft_heads_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        i, i64, sz, f, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p
        tp = ctypes.POINTER(md_tree)
        sig = {
            "md_tree_validate": ([tp, i, vp], i),
            "md_heads_weight_bytes": ([i, i, i, i, i], i64),
            "md_certified_rounding_allowance": ([i], f),
            "md_heads_fused": ([i, i, i, i, i], i),
            "md_set_wait_limits": ([i, i], i),
            "md_heads_workspace_bytes": ([i, i, i, i, i, i, i], sz),
            "md_medusa_heads": ([i, i, i, i, i, i, vp, i, tp] + [vp] * 14 + [sz, vp], i),
            "md_vocab_tile_norms_bytes": ([i, i], sz),
            "md_vocab_tile_norms": ([i, i, i, vp, vp, vp], i),
            "md_tree_build": ([tp, i, i, i, i, i, i] + [vp] * 6 + [vp], i),
            "md_attention_workspace_bytes": ([i, i, i, i, i, i, i], sz),
            "md_tree_attention": ([tp, i, i, i, i, i, i, i, vp, vp, vp, vp, f, vp, vp, sz, vp], i),
            "md_tree_attention_noalloc": ([tp, i, i, i, i, i, i, i, vp, vp, vp, vp, f, vp, vp], i),
            "md_tree_attention_noalloc_max_bytes": ([], sz),
            "md_accept_workspace_bytes": ([i, i, i], sz),
            "md_tree_accept": ([tp, i, i, i, i, i, i, i] + [vp] * 10 + [sz, vp], i),
            "md_set_vocab_timing_events": ([vp, vp], i),
            "md_last_error": ([], ctypes.c_char_p),
            "md_hbm_read_probe": ([vp, sz, vp, vp], i),
            "md_hbm_read_probe_blocks": ([], i),
            "md_target_argmax_workspace_bytes": ([i, i, i, i], sz),
            "md_target_argmax": ([i, i, i, i] + [vp] * 6 + [sz, vp], i),
            "md_tree_accept_tokens": ([tp, i, i, i, i, i, i] + [vp] * 10, i),
            "md_heads_logits_workspace_bytes": ([i, i, i, i], sz),
            "md_medusa_heads_logits": ([i, i, i, i, i, i] + [vp] * 7 + [sz, vp], i),
            "md_draft_sample_workspace_bytes": ([i, i, i, i], sz),
            "md_draft_sample": ([i, i, i, vp, f] + [vp] * 5 + [sz, vp], i),
            "md_verify_sampled_workspace_bytes": ([i, i], sz),
            "md_tree_verify_sampled": ([tp, i, i, i, i, i, i, i, f] + [vp] * 14 + [sz, vp], i),
            "md_accept_typical_workspace_bytes": ([i, i], sz),
            "md_tree_accept_typical": ([tp, i, i, i, i, i, i, i, f, f, f] + [vp] * 11 + [sz, vp], i),
            "md_operand_order_bytes": ([i, i, i], sz),
            "md_operand_order": ([i, i, i, vp, vp, vp], i),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _check(rc: int) -> None:
    if rc != MD_OK:
        raise MedusaError(rc, lib().md_last_error().decode())


def dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return MD_F32
    if t.dtype == torch.bfloat16:
        return MD_BF16
    raise TypeError("storage dtype must be float32 or bfloat16, got %s" % t.dtype)


def md_tree_validate(tree: md_tree, K: int, k_per_head: Optional[Sequence[int]] = None) -> int:
    kp = (ctypes.c_int32 * K)(*k_per_head) if k_per_head is not None else None
    return lib().md_tree_validate(ctypes.byref(tree), K, ctypes.cast(kp, ctypes.c_void_p) if kp is not None else None)


def md_last_error() -> str:
    return lib().md_last_error().decode()


def md_heads_weight_bytes(kind: int, dt: int, d: int, V: int, K: int) -> int:
    return int(lib().md_heads_weight_bytes(kind, dt, d, V, K))


def md_heads_fused(kind: int, dt: int, M: int, d: int, K: int) -> bool:
    return bool(lib().md_heads_fused(kind, dt, M, d, K))


def md_set_wait_limits(residual_polls: int, list_polls: int) -> None:
    _check(lib().md_set_wait_limits(residual_polls, list_polls))


def md_certified_rounding_allowance(d: int) -> float:
    return float(lib().md_certified_rounding_allowance(d))


def md_heads_workspace_bytes(kind: int, dt: int, M: int, d: int, V: int, K: int, kmax: int) -> int:
    return int(lib().md_heads_workspace_bytes(kind, dt, M, d, V, K, kmax))


def md_attention_workspace_bytes(dt: int, B: int, N: int, Hq: int, Hkv: int, hd: int, max_len: int) -> int:
    return int(lib().md_attention_workspace_bytes(dt, B, N, Hq, Hkv, hd, max_len))


def md_accept_workspace_bytes(B: int, N: int, V: int) -> int:
    return int(lib().md_accept_workspace_bytes(B, N, V))


def md_medusa_heads(kind, dt, M, d, V, K, k_per_head, level, tree, h, W, b, U, E, root_tok, tree_tok, topk_idx,
                    topk_val, h_res, ws, ws_bytes=None, stream=None, U_op=None, U_norms=None, W_op=None) -> None:
    """U_op / W_op: optional operand-order copies of U / W (see md_operand_order); U_norms: optional
    tile norms of U (see md_vocab_tile_norms)."""
    kp = (ctypes.c_int32 * K)(*k_per_head)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = lib().md_medusa_heads(kind, dt, M, d, V, K, ctypes.cast(kp, ctypes.c_void_p), level,
                               ctypes.byref(tree) if tree is not None else None, _p(h), _p(W), _p(b), _p(U), _p(U_op),
                               _p(U_norms), _p(W_op), _p(E), _p(root_tok), _p(tree_tok), _p(topk_idx), _p(topk_val),
                               _p(h_res), _p(ws), ws_bytes, _stream(stream))
    _check(rc)


def md_tree_build(tree, kind, B, M, K, kmax, level, topk_idx, src_row, root_tok, lens, tree_tok, tree_pos,
                  stream=None) -> None:
    rc = lib().md_tree_build(ctypes.byref(tree), kind, B, M, K, kmax, level, _p(topk_idx), _p(src_row),
                             _p(root_tok), _p(lens), _p(tree_tok), _p(tree_pos), _stream(stream))
    _check(rc)


def md_tree_attention(tree, dt, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, scale, out, ws, ws_bytes=None,
                      stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = lib().md_tree_attention(ctypes.byref(tree), dt, B, Hq, Hkv, hd, Lcap, max_len, _p(q), _p(Kc), _p(Vc),
                                 _p(lens), float(scale), _p(out), _p(ws), ws_bytes, _stream(stream))
    _check(rc)


def md_tree_attention_noalloc(tree, dt, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, scale, out,
                              stream=None) -> None:
    rc = lib().md_tree_attention_noalloc(ctypes.byref(tree), dt, B, Hq, Hkv, hd, Lcap, max_len, _p(q), _p(Kc), _p(Vc),
                                         _p(lens), float(scale), _p(out), _stream(stream))
    _check(rc)


def md_tree_attention_noalloc_max_bytes() -> int:
    return int(lib().md_tree_attention_noalloc_max_bytes())


def md_tree_accept(tree, dt, B, K, V, Hkv, hd, Lcap, logits, tree_tok, Kc, Vc, lens, accept_len, path, next_tok,
                   compact_src, ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = lib().md_tree_accept(ctypes.byref(tree), dt, B, K, V, Hkv, hd, Lcap, _p(logits), _p(tree_tok), _p(Kc),
                              _p(Vc), _p(lens), _p(accept_len), _p(path), _p(next_tok), _p(compact_src), _p(ws),
                              ws_bytes, _stream(stream))
    _check(rc)


def md_target_argmax_workspace_bytes(dt, R, d, V) -> int:
    return int(lib().md_target_argmax_workspace_bytes(dt, R, d, V))


def md_target_argmax(dt, R, d, V, H, Wt, tok, val, ws, ws_bytes=None, stream=None, Wt_op=None) -> None:
    """Wt_op: optional operand-order copy of Wt (see md_operand_order)."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().md_target_argmax(dt, R, d, V, _p(H), _p(Wt), _p(Wt_op), _p(tok), _p(val), _p(ws), ws_bytes,
                                  _stream(stream)))


def md_operand_order_bytes(nmat, rows, cols) -> int:
    return int(lib().md_operand_order_bytes(nmat, rows, cols))


def md_operand_order(nmat, rows, cols, src, dst, stream=None) -> None:
    _check(lib().md_operand_order(nmat, rows, cols, _p(src), _p(dst), _stream(stream)))


def md_vocab_tile_norms_bytes(nmat, V) -> int:
    return int(lib().md_vocab_tile_norms_bytes(nmat, V))


def md_vocab_tile_norms(nmat, V, d, U, norms, stream=None) -> None:
    _check(lib().md_vocab_tile_norms(nmat, V, d, _p(U), _p(norms), _stream(stream)))


def vocab_tile_norms(mat):
    """A new float32 device tensor [nmat, ceil(V / 256)] holding md_vocab_tile_norms of a bf16 tensor
    [V, d] or [nmat, V, d] (computed once, when weights load)."""
    import torch

    if mat.dtype != torch.bfloat16 or mat.dim() not in (2, 3):
        raise MedusaError(MD_EINVAL, "tile norms take a bf16 [V, d] or [nmat, V, d] tensor")
    m3 = mat if mat.dim() == 3 else mat.unsqueeze(0)
    nmat, V, d = m3.shape
    out = torch.empty(md_vocab_tile_norms_bytes(nmat, V) // 4, dtype=torch.float32, device=mat.device)
    md_vocab_tile_norms(nmat, V, d, m3.contiguous(), out)
    return out.view(nmat, -1)


def operand_order(mat):
    """A new device tensor holding the operand-order copy of a bf16 tensor
    [rows, cols] or [nmat, rows, cols] (allocated once, when weights load)."""
    import torch

    if mat.dtype != torch.bfloat16 or mat.dim() not in (2, 3):
        raise MedusaError(MD_EINVAL, "operand order takes a bf16 [rows, cols] or [nmat, rows, cols] tensor")
    m3 = mat if mat.dim() == 3 else mat.unsqueeze(0)
    nmat, rows, cols = m3.shape
    n = md_operand_order_bytes(nmat, rows, cols)
    if n == 0:
        raise MedusaError(MD_EUNSUPPORTED, "operand order needs cols a positive multiple of 32 (got %d)" % cols)
    dst = torch.empty(n // 2, dtype=torch.bfloat16, device=mat.device)
    md_operand_order(nmat, rows, cols, m3.contiguous(), dst)
    return dst


def md_tree_accept_tokens(tree, dt, B, K, Hkv, hd, Lcap, target_tok, tree_tok, Kc, Vc, lens, accept_len, path,
                          next_tok, compact_src, stream=None) -> None:
    rc = lib().md_tree_accept_tokens(ctypes.byref(tree), dt, B, K, Hkv, hd, Lcap, _p(target_tok), _p(tree_tok), _p(Kc),
                                     _p(Vc), _p(lens), _p(accept_len), _p(path), _p(next_tok), _p(compact_src),
                                     _stream(stream))
    _check(rc)


def md_heads_logits_workspace_bytes(kind: int, M: int, d: int, K: int) -> int:
    return int(lib().md_heads_logits_workspace_bytes(kind, M, d, K))


def md_medusa_heads_logits(kind, dt, M, d, V, K, h, W, b, U, logits, h_res, ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().md_medusa_heads_logits(kind, dt, M, d, V, K, _p(h), _p(W), _p(b), _p(U), _p(logits), _p(h_res),
                                        _p(ws), ws_bytes, _stream(stream)))


def md_draft_sample_workspace_bytes(M: int, K: int, V: int, kmax: int) -> int:
    return int(lib().md_draft_sample_workspace_bytes(M, K, V, kmax))


def md_draft_sample(M, K, V, k_per_head, temperature, logits, words, tok, lse, ws, ws_bytes=None, stream=None) -> None:
    kp = (ctypes.c_int32 * K)(*k_per_head)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().md_draft_sample(M, K, V, ctypes.cast(kp, ctypes.c_void_p), float(temperature), _p(logits), _p(words),
                                 _p(tok), _p(lse), _p(ws), ws_bytes, _stream(stream)))


def md_verify_sampled_workspace_bytes(B: int, N: int) -> int:
    return int(lib().md_verify_sampled_workspace_bytes(B, N))


def md_tree_verify_sampled(tree, dt, B, K, V, Hkv, hd, Lcap, temperature, target_logits, head_logits, head_lse,
                           tree_tok, u_words, g_words, Kc, Vc, lens, accept_len, path, next_tok, compact_src, ws,
                           ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().md_tree_verify_sampled(ctypes.byref(tree), dt, B, K, V, Hkv, hd, Lcap, float(temperature),
                                        _p(target_logits), _p(head_logits), _p(head_lse), _p(tree_tok), _p(u_words),
                                        _p(g_words), _p(Kc), _p(Vc), _p(lens), _p(accept_len), _p(path), _p(next_tok),
                                        _p(compact_src), _p(ws), ws_bytes, _stream(stream)))


def md_accept_typical_workspace_bytes(B: int, N: int) -> int:
    return int(lib().md_accept_typical_workspace_bytes(B, N))


def md_tree_accept_typical(tree, dt, B, K, V, Hkv, hd, Lcap, temperature, eps, delta, target_logits, tree_tok, g_words,
                           Kc, Vc, lens, accept_len, path, next_tok, compact_src, ws, ws_bytes=None,
                           stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().md_tree_accept_typical(ctypes.byref(tree), dt, B, K, V, Hkv, hd, Lcap, float(temperature),
                                        float(eps), float(delta), _p(target_logits), _p(tree_tok), _p(g_words), _p(Kc),
                                        _p(Vc), _p(lens), _p(accept_len), _p(path), _p(next_tok), _p(compact_src),
                                        _p(ws), ws_bytes, _stream(stream)))


def md_set_vocab_timing_events(start, stop) -> None:
    """start/stop: raw hipEvent_t handles (ints) or None."""
    _check(lib().md_set_vocab_timing_events(start, stop))


def md_hbm_read_probe_blocks() -> int:
    return int(lib().md_hbm_read_probe_blocks())


def md_hbm_read_probe(buf, nbytes: int, sink, stream=None) -> None:
    _check(lib().md_hbm_read_probe(_p(buf), nbytes, _p(sink), _stream(stream)))
