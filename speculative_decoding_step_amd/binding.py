"""ctypes binding of libeagle3.so: the C ABI in include/eagle3.h, same names.

Argument marshalling only.  Device pointers are passed as integers (for
example ``tensor.data_ptr()``) or None for NULL; every nonzero status raises
:class:`Eagle3Error`.  The library must exist (``python -m
speculative_decoding_step_amd.build``); nothing here falls back to another
implementation.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libeagle3.so")

F32, BF16 = 0, 1
GREEDY_TREE, SAMPLE_CHAIN, SAMPLE_TREE = 0, 1, 2
LM_ALL, LM_LAST, LM_NONE = 0, 1, 2
PROF_GEMM_M64, PROF_GEMM_M16, PROF_ATTN, PROF_GEMM_BIG = 0, 1, 2, 3
DEV_KV_OVERFLOW, DEV_BAD_TREE, DEV_BAD_TOKEN, DEV_BAD_PATH = 1, 2, 4, 8

EXPORTS = [
    "eagle3_kv_bytes", "eagle3_workspace_bytes", "eagle3_create", "eagle3_destroy", "eagle3_verify_tree",
    "eagle3_draft_prefill", "eagle3_draft_tree", "eagle3_tree_from_logits", "eagle3_accept", "eagle3_compact_kv",
    "eagle3_sample", "eagle3_set_stream", "eagle3_status_string", "eagle3_device_status", "eagle3_profile", "eagle3_profile_read",
    "eagle3_pack_linear", "eagle3_ttt_workspace_bytes", "eagle3_ttt_attention", "eagle3_paged_kv_bytes",
    "eagle3_create_paged", "eagle3_set_draft_lengths", "eagle3_spec_decode_metadata", "eagle3_set_draft_logits_out",
    "eagle3_set_hidden_out", "eagle3_ttt_attention_static",
]


class Eagle3Error(RuntimeError):
    pass


class Shape(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32),
                ("rope_theta", C.c_float), ("rms_eps", C.c_float), ("dtype", C.c_int32), ("taps", C.c_int32 * 3),
                ("draft_vocab", C.c_int32)]


class SpecCfg(C.Structure):
    _fields_ = [("mode", C.c_int32), ("depth", C.c_int32), ("topk", C.c_int32), ("n_nodes", C.c_int32),
                ("temperature", C.c_float), ("draft_greedy", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")]


class TargetWeights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("layers", C.POINTER(LayerWeights)), ("final_norm", C.c_void_p),
                ("lm_head", C.c_void_p)]


class HeadWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("fc", "input_norm", "hidden_norm", "wq", "wk", "wv", "wo", "post_norm", "w_gate", "w_up",
                 "w_down", "final_norm", "lm_head", "d2t")]


class KvPages(C.Structure):
    _fields_ = [("block_size", C.c_int32), ("n_blocks", C.c_int32), ("blocks_per_seq", C.c_int32),
                ("block_table", C.c_void_p)]


_lib = None
P = C.c_void_p
I32 = C.c_int32


def lib():
    """Load libeagle3.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Eagle3Error(f"{LIB_PATH} is missing: build it with python -m speculative_decoding_step_amd.build")
        L = C.CDLL(LIB_PATH)
        sig = {
            "eagle3_kv_bytes": [C.POINTER(Shape), I32, I32, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)],
            "eagle3_workspace_bytes": [C.POINTER(Shape), C.POINTER(SpecCfg), I32, I32, I32, C.POINTER(C.c_size_t)],
            "eagle3_create": [C.POINTER(Shape), C.POINTER(SpecCfg), C.POINTER(TargetWeights), C.POINTER(HeadWeights),
                              I32, I32, I32, P, C.c_size_t, P, P, P, C.POINTER(P)],
            "eagle3_destroy": [P],
            "eagle3_paged_kv_bytes": [C.POINTER(Shape), I32, I32, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)],
            "eagle3_create_paged": [C.POINTER(Shape), C.POINTER(SpecCfg), C.POINTER(TargetWeights),
                                    C.POINTER(HeadWeights), I32, I32, C.POINTER(KvPages), P, C.c_size_t, P, P, P,
                                    C.POINTER(P)],
            "eagle3_set_draft_lengths": [P, P],
            "eagle3_spec_decode_metadata": [I32, I32, P, P, P, P, P, P, P, P, P, P],
            "eagle3_pack_linear": [I32, P, P, I32, I32, P],
            "eagle3_verify_tree": [P, I32, I32, P, I32, P, P, P, I32, P, P, P, P],
            "eagle3_draft_prefill": [P, I32, I32, P, I32, P, P],
            "eagle3_draft_tree": [P, I32, P, P, P, P, P, P, P, P, P, P, P, P],
            "eagle3_tree_from_logits": [P, I32, P, P, P, P, P, P, P, P, P, P, P],
            "eagle3_accept": [P, I32, I32, P, P, P, P, P, P, P, P, P, P],
            "eagle3_compact_kv": [P, I32, P, I32, P, P, P, P, P, P, P, P, P],
            "eagle3_set_draft_logits_out": [P, P],
            "eagle3_set_hidden_out": [P, P],
            "eagle3_ttt_attention_static": [I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P],
            "eagle3_sample": [P, I32, P, C.c_float, P, P],
            "eagle3_ttt_workspace_bytes": [I32, I32, I32, C.POINTER(C.c_size_t)],
            "eagle3_ttt_attention": [I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, C.c_size_t, P],
            "eagle3_set_stream": [P, P],
            "eagle3_device_status": [P, C.POINTER(I32)],
            "eagle3_profile": [P, I32],
            "eagle3_profile_read": [P, I32, C.POINTER(C.c_int64), C.POINTER(C.c_double), C.POINTER(C.c_double),
                                    C.POINTER(C.c_double)],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = C.c_int
        L.eagle3_status_string.argtypes = [C.c_int]
        L.eagle3_status_string.restype = C.c_char_p
        _lib = L
    return _lib


def _check(st: int, what: str):
    if st != 0:
        raise Eagle3Error(f"{what}: {lib().eagle3_status_string(st).decode()} ({st})")


def eagle3_status_string(st: int) -> str:
    return lib().eagle3_status_string(st).decode()


def eagle3_kv_bytes(shape: Shape, max_batch: int, max_seq: int):
    t, d = C.c_size_t(), C.c_size_t()
    _check(lib().eagle3_kv_bytes(C.byref(shape), max_batch, max_seq, C.byref(t), C.byref(d)), "eagle3_kv_bytes")
    return t.value, d.value


def eagle3_workspace_bytes(shape: Shape, cfg: SpecCfg, max_batch: int, max_rows: int, max_seq: int) -> int:
    n = C.c_size_t()
    _check(lib().eagle3_workspace_bytes(C.byref(shape), C.byref(cfg), max_batch, max_rows, max_seq, C.byref(n)),
           "eagle3_workspace_bytes")
    return n.value


def eagle3_create(shape: Shape, cfg: SpecCfg, target: TargetWeights, head: HeadWeights, max_batch: int,
                  max_rows: int, max_seq: int, workspace: int, workspace_bytes: int, kv_target: int, kv_draft: int,
                  stream: int) -> int:
    out = P()
    _check(lib().eagle3_create(C.byref(shape), C.byref(cfg), C.byref(target), C.byref(head), max_batch, max_rows,
                               max_seq, workspace, workspace_bytes, kv_target, kv_draft, stream, C.byref(out)),
           "eagle3_create")
    return out.value


def eagle3_paged_kv_bytes(shape: Shape, block_size: int, n_blocks: int):
    t, d = C.c_size_t(), C.c_size_t()
    _check(lib().eagle3_paged_kv_bytes(C.byref(shape), block_size, n_blocks, C.byref(t), C.byref(d)),
           "eagle3_paged_kv_bytes")
    return t.value, d.value


def eagle3_create_paged(shape: Shape, cfg: SpecCfg, target: TargetWeights, head: HeadWeights, max_batch: int,
                        max_rows: int, pages: KvPages, workspace: int, workspace_bytes: int, kv_target: int,
                        kv_draft: int, stream: int) -> int:
    out = P()
    _check(lib().eagle3_create_paged(C.byref(shape), C.byref(cfg), C.byref(target), C.byref(head), max_batch,
                                     max_rows, C.byref(pages), workspace, workspace_bytes, kv_target, kv_draft, stream,
                                     C.byref(out)), "eagle3_create_paged")
    return out.value


def eagle3_set_draft_lengths(ctx, n_draft):
    _check(lib().eagle3_set_draft_lengths(ctx, n_draft), "eagle3_set_draft_lengths")


def eagle3_spec_decode_metadata(batch, max_drafts, cu_num_scheduled_tokens, num_draft_tokens, input_ids,
                                cu_num_draft_tokens, logits_indices, target_logits_indices, bonus_logits_indices,
                                draft_token_ids, error, stream):
    _check(lib().eagle3_spec_decode_metadata(batch, max_drafts, cu_num_scheduled_tokens, num_draft_tokens, input_ids,
                                             cu_num_draft_tokens, logits_indices, target_logits_indices,
                                             bonus_logits_indices, draft_token_ids, error, stream),
           "eagle3_spec_decode_metadata")


def eagle3_destroy(ctx: int):
    _check(lib().eagle3_destroy(ctx), "eagle3_destroy")


def eagle3_pack_linear(dtype: int, src: int, dst: int, rows: int, cols: int, stream: int):
    _check(lib().eagle3_pack_linear(dtype, src, dst, rows, cols, stream), "eagle3_pack_linear")


def eagle3_verify_tree(ctx, seq_begin, batch, seq_lens, n_rows, tokens, pos, mask, lm_mode, logits, argmax, margin,
                       aux):
    _check(lib().eagle3_verify_tree(ctx, seq_begin, batch, seq_lens, n_rows, tokens, pos, mask, lm_mode, logits,
                                    argmax, margin, aux), "eagle3_verify_tree")


def eagle3_draft_prefill(ctx, seq_begin, batch, start, n_rows, aux, next_tok):
    _check(lib().eagle3_draft_prefill(ctx, seq_begin, batch, start, n_rows, aux, next_tok), "eagle3_draft_prefill")


def eagle3_draft_tree(ctx, batch, seq_lens, new_len, aux_new, next_tok, uniforms, tokens, parents, depth, pos, mask,
                      score, q):
    _check(lib().eagle3_draft_tree(ctx, batch, seq_lens, new_len, aux_new, next_tok, uniforms, tokens, parents, depth,
                                   pos, mask, score, q), "eagle3_draft_tree")


def eagle3_tree_from_logits(ctx, batch, roots, seq_lens, logits_table, uniforms, tokens, parents, depth, pos, mask,
                            score, q):
    _check(lib().eagle3_tree_from_logits(ctx, batch, roots, seq_lens, logits_table, uniforms, tokens, parents, depth,
                                         pos, mask, score, q), "eagle3_tree_from_logits")


def eagle3_accept(ctx, batch, n_rows, tokens, parents, argmax, logits, q, uniforms, path, path_len, next_root,
                  emitted):
    _check(lib().eagle3_accept(ctx, batch, n_rows, tokens, parents, argmax, logits, q, uniforms, path, path_len,
                               next_root, emitted), "eagle3_accept")


def eagle3_compact_kv(ctx, batch, seq_lens, n_rows, path, path_len, tokens, next_root, aux_tree, aux_new, next_tok,
                      new_len, src_dst=None):
    _check(lib().eagle3_compact_kv(ctx, batch, seq_lens, n_rows, path, path_len, tokens, next_root, aux_tree, aux_new,
                                   next_tok, new_len, src_dst), "eagle3_compact_kv")


def eagle3_set_hidden_out(ctx, buf):
    _check(lib().eagle3_set_hidden_out(ctx, buf), "eagle3_set_hidden_out")


def eagle3_set_draft_logits_out(ctx, table):
    _check(lib().eagle3_set_draft_logits_out(ctx, table), "eagle3_set_draft_logits_out")


def eagle3_sample(ctx, n, logits, temperature, uniforms, tokens):
    _check(lib().eagle3_sample(ctx, n, logits, temperature, uniforms, tokens), "eagle3_sample")


def eagle3_ttt_workspace_bytes(T, n_heads, head_dim) -> int:
    b = C.c_size_t()
    _check(lib().eagle3_ttt_workspace_bytes(T, n_heads, head_dim, C.byref(b)), "eagle3_ttt_workspace_bytes")
    return b.value


def eagle3_ttt_attention(dtype, T, S, n_heads, n_kv_heads, head_dim, q, k0, v0, ks, vs, out, ws, ws_bytes, stream):
    _check(lib().eagle3_ttt_attention(dtype, T, S, n_heads, n_kv_heads, head_dim, q, k0, v0, ks, vs, out, ws,
                                      ws_bytes, stream), "eagle3_ttt_attention")


def eagle3_ttt_attention_static(dtype, T, S, n_heads, n_kv_heads, head_dim, q, k0, v0, ks, vs, out, stream):
    _check(lib().eagle3_ttt_attention_static(dtype, T, S, n_heads, n_kv_heads, head_dim, q, k0, v0, ks, vs, out,
                                             stream), "eagle3_ttt_attention_static")


def eagle3_set_stream(ctx, stream):
    _check(lib().eagle3_set_stream(ctx, stream), "eagle3_set_stream")


def eagle3_device_status(ctx) -> int:
    f = I32()
    _check(lib().eagle3_device_status(ctx, C.byref(f)), "eagle3_device_status")
    return f.value


def eagle3_profile(ctx, enable: bool):
    _check(lib().eagle3_profile(ctx, 1 if enable else 0), "eagle3_profile")


def eagle3_profile_read(ctx, kernel: int):
    n, ms, by, fl = C.c_int64(), C.c_double(), C.c_double(), C.c_double()
    _check(lib().eagle3_profile_read(ctx, kernel, C.byref(n), C.byref(ms), C.byref(by), C.byref(fl)),
           "eagle3_profile_read")
    return n.value, ms.value, by.value, fl.value
