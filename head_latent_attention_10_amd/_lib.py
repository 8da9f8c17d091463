"""ctypes binding of libmla_hip.so: argument marshalling only.

Every function here has the name of the C entry point it calls and takes the
same arguments; tensors may be torch tensors (their data pointer is passed) or
plain integer device addresses.  No arithmetic of the decode step happens in
Python.  If the HIP library has not been built, loading raises instead of
falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_hip.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = 0, -1, -2, -3, -4
MLA_F32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2
DTYPE_CODES = {"f32": MLA_F32, "bf16": MLA_BF16, "e4m3": MLA_FP8_E4M3}


class MlaDecodeParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("d_nope", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32),
        ("rope_dtype", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
    ]


class MlaCacheWriteParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("d_model", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("x_dtype", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32),
        ("rope_dtype", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("rope_base", ctypes.c_float),
    ]


class MlaDsaParams(ctypes.Structure):
    _fields_ = [
        ("index_heads", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32),
    ]


class MlaTplaParams(ctypes.Structure):
    _fields_ = [
        ("shards", ctypes.c_int32),
        ("mu", ctypes.c_float * 4),
    ]


class MlaError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_PP = ctypes.POINTER(MlaDecodeParams)
_WP = ctypes.POINTER(MlaCacheWriteParams)
_DP = ctypes.POINTER(MlaDsaParams)
_TP = ctypes.POINTER(MlaTplaParams)
_I32 = ctypes.c_int32

_SIGNATURES = {
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_decode_workspace_size": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_decode_num_splits": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_int32)]),
    "mla_absorbed_dtype": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_int32)]),
    "mla_decode": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "mla_decode_no_alloc": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "mla_decode_timed": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P]),
    "mla_absorb_q": (ctypes.c_int, [_PP, _P, _P, _P, _P]),
    "mla_attend_latent": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "mla_attend_partial": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "mla_combine": (ctypes.c_int, [_PP, _P, _P, ctypes.c_size_t, _P]),
    "mla_partials_layout": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_int32)]),
    "mla_up_project": (ctypes.c_int, [_PP, _P, _P, _P, _P]),
    "mla_gather_cache": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P]),
    "mla_split_begin": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
    "mla_split_owner": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64]),
    "mla_split_plan": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p]),
    "mla_cache_write_workspace_size": (ctypes.c_int, [_WP, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_cache_write": (ctypes.c_int, [_WP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "mla_quantize_e4m3_rows": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]),
    "mla_indexer_scores": (ctypes.c_int, [_PP, _DP, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P]),
    "mla_topk_select": (ctypes.c_int, [_P, _I32, _P, _I32, _I32, _P, _I32, _P, _P]),
    "mla_topk_select_split_workspace_size": (ctypes.c_int,
                                             [_I32, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_topk_select_split": (ctypes.c_int, [_P, _I32, _P, _I32, _I32, _P, _I32, _P, _P,
                                             ctypes.c_size_t, _P]),
    "mla_decode_sparse_workspace_size": (ctypes.c_int, [_PP, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_decode_sparse": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]),
    "mla_dsa_decode_workspace_size": (ctypes.c_int, [_PP, _DP, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_tpla_decode_workspace_size": (ctypes.c_int, [_PP, _TP, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_grouped_decode": (ctypes.c_int, [_PP, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "mla_prefill_workspace_size": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_prefill": (ctypes.c_int, [_PP, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P]),
    "mla_tpla_decode": (ctypes.c_int, [_PP, _TP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
    "mla_dsa_decode": (ctypes.c_int, [_PP, _DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _P, _P, ctypes.c_size_t, _P]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m head_latent_attention_10_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    return list(_SIGNATURES)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, st: int):
    if st != MLA_OK:
        lib = load_library()
        raise MlaError(st, fn, lib.mla_last_error().decode())


def make_params(batch, num_heads, d_nope, d_rope, d_latent, d_v, page_size, max_blocks_per_seq,
                num_blocks, q_dtype="bf16", cache_dtype="bf16", rope_dtype="bf16",
                weight_dtype="bf16", out_dtype="bf16", sm_scale=0.0, num_splits=0):
    code = lambda d: DTYPE_CODES[d] if isinstance(d, str) else int(d)
    return MlaDecodeParams(batch, num_heads, d_nope, d_rope, d_latent, d_v, page_size,
                           max_blocks_per_seq, num_blocks, code(q_dtype), code(cache_dtype),
                           code(rope_dtype), code(weight_dtype), code(out_dtype), float(sm_scale),
                           num_splits)


def mla_status_string(status: int) -> str:
    return load_library().mla_status_string(status).decode()


def mla_last_error() -> str:
    return load_library().mla_last_error().decode()


def mla_decode_workspace_size(p: MlaDecodeParams) -> int:
    n = ctypes.c_size_t(0)
    _check("mla_decode_workspace_size", load_library().mla_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def mla_decode_num_splits(p: MlaDecodeParams) -> int:
    n = ctypes.c_int32(0)
    _check("mla_decode_num_splits", load_library().mla_decode_num_splits(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def mla_absorbed_dtype(p: MlaDecodeParams) -> int:
    n = ctypes.c_int32(0)
    _check("mla_absorbed_dtype", load_library().mla_absorbed_dtype(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def mla_decode(p, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, W_UK, W_UV, out,
               workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("mla_decode", load_library().mla_decode(
        ctypes.byref(p), _ptr(q), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope), _ptr(block_table),
        _ptr(seq_lens), _ptr(W_UK), _ptr(W_UV), _ptr(out), _ptr(workspace), workspace_bytes,
        _stream(stream)))


def mla_decode_timed(p, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, W_UK, W_UV, out,
                     workspace, workspace_bytes, stream, ev_before, ev_after):
    """ev_before / ev_after: torch.cuda.Event (created with enable_timing) or raw hipEvent_t."""
    evb = ev_before.cuda_event if hasattr(ev_before, "cuda_event") else ev_before
    eva = ev_after.cuda_event if hasattr(ev_after, "cuda_event") else ev_after
    _check("mla_decode_timed", load_library().mla_decode_timed(
        ctypes.byref(p), _ptr(q), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope), _ptr(block_table),
        _ptr(seq_lens), _ptr(W_UK), _ptr(W_UV), _ptr(out), _ptr(workspace), workspace_bytes,
        _stream(stream), evb, eva))


# Size of the fixed device array mla_decode_no_alloc works in (the header's
# MLA_NO_ALLOC_SCRATCH_BYTES).
MLA_NO_ALLOC_SCRATCH_BYTES = 128 << 20


def mla_decode_no_alloc(p, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, W_UK, W_UV, out,
                        stream=None):
    _check("mla_decode_no_alloc", load_library().mla_decode_no_alloc(
        ctypes.byref(p), _ptr(q), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope), _ptr(block_table),
        _ptr(seq_lens), _ptr(W_UK), _ptr(W_UV), _ptr(out), _stream(stream)))


def mla_absorb_q(p, q, W_UK, q_lat, stream=None):
    _check("mla_absorb_q", load_library().mla_absorb_q(
        ctypes.byref(p), _ptr(q), _ptr(W_UK), _ptr(q_lat), _stream(stream)))


def mla_attend_latent(p, q_lat, c_kv, c_kv_scale, k_rope, block_table, seq_lens, o_lat,
                      workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("mla_attend_latent", load_library().mla_attend_latent(
        ctypes.byref(p), _ptr(q_lat), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope),
        _ptr(block_table), _ptr(seq_lens), _ptr(o_lat), _ptr(workspace), workspace_bytes,
        _stream(stream)))


def mla_attend_partial(p, q_lat, c_kv, c_kv_scale, k_rope, block_table, seq_lens, workspace,
                       workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("mla_attend_partial", load_library().mla_attend_partial(
        ctypes.byref(p), _ptr(q_lat), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope),
        _ptr(block_table), _ptr(seq_lens), _ptr(workspace), workspace_bytes, _stream(stream)))


def mla_combine(p, o_lat, workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("mla_combine", load_library().mla_combine(
        ctypes.byref(p), _ptr(o_lat), _ptr(workspace), workspace_bytes, _stream(stream)))


def mla_partials_layout(p):
    """(part_o byte offset, part_lse byte offset, slots, bf16_rows) of the
    partials mla_attend_partial writes into the workspace for *p; the partial
    outputs are row-major [slot][head][d_latent], bf16 when bf16_rows is 1,
    else fp32."""
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    n, f = ctypes.c_int32(), ctypes.c_int32()
    _check("mla_partials_layout", load_library().mla_partials_layout(
        ctypes.byref(p), ctypes.byref(a), ctypes.byref(b), ctypes.byref(n), ctypes.byref(f)))
    return a.value, b.value, n.value, f.value


def mla_up_project(p, o_lat, W_UV, out, stream=None):
    _check("mla_up_project", load_library().mla_up_project(
        ctypes.byref(p), _ptr(o_lat), _ptr(W_UV), _ptr(out), _stream(stream)))


def mla_gather_cache(p, c_kv, c_kv_scale, k_rope, block_table, seq_lens, max_tokens, c_out,
                     scale_out, rope_out, stream=None):
    _check("mla_gather_cache", load_library().mla_gather_cache(
        ctypes.byref(p), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope), _ptr(block_table),
        _ptr(seq_lens), int(max_tokens), _ptr(c_out), _ptr(scale_out), _ptr(rope_out),
        _stream(stream)))


def mla_split_begin(n_tiles: int, splits: int, g: int) -> int:
    return load_library().mla_split_begin(n_tiles, splits, g)


def mla_split_owner(n_tiles: int, splits: int, tile: int) -> int:
    return load_library().mla_split_owner(n_tiles, splits, tile)


def mla_split_plan(tiles, splits: int):
    """Host split plan for tiles per sequence -> (split_first [splits + 1],
    seq_splits [batch, 2]) as int32 numpy arrays."""
    import numpy as np
    t = np.ascontiguousarray(np.asarray(tiles, dtype=np.int32))
    first = np.zeros(int(splits) + 1, dtype=np.int32)
    seq = np.zeros((len(t), 2), dtype=np.int32)
    _check("mla_split_plan", load_library().mla_split_plan(
        t.ctypes.data, len(t), int(splits), first.ctypes.data, seq.ctypes.data))
    return first, seq


def make_write_params(batch, d_model, d_latent, d_rope, page_size, max_blocks_per_seq, num_blocks,
                      x_dtype="bf16", weight_dtype="bf16", cache_dtype="bf16", rope_dtype="bf16",
                      rms_eps=1e-6, rope_base=10000.0):
    code = lambda d: DTYPE_CODES[d] if isinstance(d, str) else int(d)
    return MlaCacheWriteParams(batch, d_model, d_latent, d_rope, page_size, max_blocks_per_seq,
                               num_blocks, code(x_dtype), code(weight_dtype), code(cache_dtype),
                               code(rope_dtype), float(rms_eps), float(rope_base))


def mla_cache_write_workspace_size(p: MlaCacheWriteParams) -> int:
    n = ctypes.c_size_t(0)
    _check("mla_cache_write_workspace_size",
           load_library().mla_cache_write_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def mla_cache_write(p, x, W_DKV, gamma, W_KR, positions, block_table, c_kv, c_kv_scale, k_rope,
                    workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_cache_write", load_library().mla_cache_write(
        ctypes.byref(p), _ptr(x), _ptr(W_DKV), _ptr(gamma), _ptr(W_KR), _ptr(positions),
        _ptr(block_table), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope), _ptr(workspace),
        workspace_bytes, _stream(stream)))


def mla_quantize_e4m3_rows(x, rows: int, d: int, codes, scales, stream=None):
    _check("mla_quantize_e4m3_rows", load_library().mla_quantize_e4m3_rows(
        _ptr(x), int(rows), int(d), _ptr(codes), _ptr(scales), _stream(stream)))


# ------------------------------------------------------------------ DSA

def make_dsa_params(index_heads=64, index_dim=128, topk=2048) -> MlaDsaParams:
    return MlaDsaParams(int(index_heads), int(index_dim), int(topk))


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


def mla_indexer_scores(p, d, q_I, q_I_scale, w_I, k_I, k_I_scale, block_table, seq_lens, scores,
                       score_stride: int, stream=None):
    _check("mla_indexer_scores", load_library().mla_indexer_scores(
        ctypes.byref(p), ctypes.byref(d), _ptr(q_I), _ptr(q_I_scale), _ptr(w_I), _ptr(k_I),
        _ptr(k_I_scale), _ptr(block_table), _ptr(seq_lens), _ptr(scores), int(score_stride),
        _stream(stream)))


def mla_topk_select(scores, score_stride: int, seq_lens, batch: int, k: int, indices,
                    index_stride: int, counts, stream=None):
    _check("mla_topk_select", load_library().mla_topk_select(
        _ptr(scores), int(score_stride), _ptr(seq_lens), int(batch), int(k), _ptr(indices),
        int(index_stride), _ptr(counts), _stream(stream)))


def mla_topk_select_split_workspace_size(batch: int, score_stride: int) -> int:
    n = ctypes.c_size_t(0)
    _check("mla_topk_select_split_workspace_size",
           load_library().mla_topk_select_split_workspace_size(int(batch), int(score_stride),
                                                               ctypes.byref(n)))
    return n.value


def mla_topk_select_split(scores, score_stride: int, seq_lens, batch: int, k: int, indices,
                          index_stride: int, counts, workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace)
    _check("mla_topk_select_split", load_library().mla_topk_select_split(
        _ptr(scores), int(score_stride), _ptr(seq_lens), int(batch), int(k), _ptr(indices),
        int(index_stride), _ptr(counts), _ptr(workspace), workspace_bytes, _stream(stream)))


def mla_decode_sparse_workspace_size(p, index_stride: int) -> int:
    n = ctypes.c_size_t(0)
    _check("mla_decode_sparse_workspace_size", load_library().mla_decode_sparse_workspace_size(
        ctypes.byref(p), int(index_stride), ctypes.byref(n)))
    return n.value


def mla_decode_sparse(p, q, c_kv, c_kv_scale, k_rope, block_table, indices, index_stride: int,
                      counts, W_UK, W_UV, out, workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace)
    _check("mla_decode_sparse", load_library().mla_decode_sparse(
        ctypes.byref(p), _ptr(q), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope), _ptr(block_table),
        _ptr(indices), int(index_stride), _ptr(counts), _ptr(W_UK), _ptr(W_UV), _ptr(out),
        _ptr(workspace), workspace_bytes, _stream(stream)))


def mla_dsa_decode_workspace_size(p, d) -> int:
    n = ctypes.c_size_t(0)
    _check("mla_dsa_decode_workspace_size", load_library().mla_dsa_decode_workspace_size(
        ctypes.byref(p), ctypes.byref(d), ctypes.byref(n)))
    return n.value


def mla_dsa_decode(p, d, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, q_I, q_I_scale, w_I,
                   k_I, k_I_scale, W_UK, W_UV, out, indices_out, workspace, workspace_bytes=None,
                   stream=None):
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace)
    _check("mla_dsa_decode", load_library().mla_dsa_decode(
        ctypes.byref(p), ctypes.byref(d), _ptr(q), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope),
        _ptr(block_table), _ptr(seq_lens), _ptr(q_I), _ptr(q_I_scale), _ptr(w_I), _ptr(k_I),
        _ptr(k_I_scale), _ptr(W_UK), _ptr(W_UV), _ptr(out), _ptr(indices_out), _ptr(workspace),
        workspace_bytes, _stream(stream)))


# ------------------------------------------------------------------ TPLA

def make_tpla_params(shards=2, mu=None) -> MlaTplaParams:
    mu = [1.0] * 4 if mu is None else list(mu) + [1.0] * (4 - len(mu))
    return MlaTplaParams(int(shards), (ctypes.c_float * 4)(*[float(x) for x in mu[:4]]))


def mla_tpla_decode_workspace_size(p, t) -> int:
    n = ctypes.c_size_t(0)
    _check("mla_tpla_decode_workspace_size", load_library().mla_tpla_decode_workspace_size(
        ctypes.byref(p), ctypes.byref(t), ctypes.byref(n)))
    return n.value


def mla_tpla_decode(p, t, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, W_UK, W_UV, out,
                    workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace)
    _check("mla_tpla_decode", load_library().mla_tpla_decode(
        ctypes.byref(p), ctypes.byref(t), _ptr(q), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope),
        _ptr(block_table), _ptr(seq_lens), _ptr(W_UK), _ptr(W_UV), _ptr(out), _ptr(workspace),
        workspace_bytes, _stream(stream)))


# ------------------------------------------------------------------ grouped MLA

def mla_grouped_decode(p, latent_groups: int, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens,
                       W_UK, W_UV, out, workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace)
    _check("mla_grouped_decode", load_library().mla_grouped_decode(
        ctypes.byref(p), int(latent_groups), _ptr(q), _ptr(c_kv), _ptr(c_kv_scale), _ptr(k_rope),
        _ptr(block_table), _ptr(seq_lens), _ptr(W_UK), _ptr(W_UV), _ptr(out), _ptr(workspace),
        workspace_bytes, _stream(stream)))


# ------------------------------------------------------------------ prefill

# The workspace mla_prefill_workspace_size asks for at most (the header's
# MLA_PREFILL_DEFAULT_WORKSPACE_BYTES); any workspace of one (sequence, head)
# unit or more works, the call then running in chunks of units.
MLA_PREFILL_DEFAULT_WORKSPACE_BYTES = 1 << 30


def prefill_unit_bytes(max_blocks_per_seq: int, page_size: int) -> int:
    """Workspace bytes of one (sequence, head) unit of mla_prefill: its keys
    (192 wide) and values (128 wide) in bf16 over Tpad tokens, Tpad the cache
    capacity of a sequence rounded up to 128."""
    tpad = -(-max_blocks_per_seq * page_size // 128) * 128
    return tpad * (192 + 128) * 2


def mla_prefill_workspace_size(p) -> int:
    n = ctypes.c_size_t(0)
    _check("mla_prefill_workspace_size",
           load_library().mla_prefill_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def mla_prefill(p, max_q_len: int, q, q_lens, c_kv, c_kv_scale, k_rope, block_table, seq_lens,
                W_UK, W_UV, out, workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace)
    _check("mla_prefill", load_library().mla_prefill(
        ctypes.byref(p), int(max_q_len), _ptr(q), _ptr(q_lens), _ptr(c_kv), _ptr(c_kv_scale),
        _ptr(k_rope),
        _ptr(block_table), _ptr(seq_lens), _ptr(W_UK), _ptr(W_UV), _ptr(out), _ptr(workspace),
        workspace_bytes, _stream(stream)))
