"""ctypes binding of libmla_amd.so: argument marshalling only.

Every function here has the name of the C entry point it calls (include/mla.h)
and does nothing but turn torch tensors into pointers, sizes and dtype codes,
call the library, and raise MlaError on a non-zero status.  All computation
happens in the HIP kernels behind the C ABI; torch only owns device memory and
streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Union

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_AMD_LIB names another build of the same library (the host-sanitized
# build that the sanitizer test loads); by default the in-tree build.
LIB_PATH = os.environ.get("MLA_AMD_LIB") or os.path.join(_HERE, "libmla_amd.so")

MLA_F32, MLA_BF16 = 0, 1
MLA_OK, MLA_ERR_NULL, MLA_ERR_DIMS, MLA_ERR_SHAPE = 0, 1, 2, 3
MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP, MLA_ERR_ARG = 4, 5, 6, 7
MLA_DATA_NEG_LEN, MLA_DATA_LEN_OVER_TABLE, MLA_DATA_LEN_BELOW_TQ, MLA_DATA_BAD_BLOCK = 1, 2, 4, 8
MLA_DATA_BAD_SLOT = 0x10
MLA_ROPE_NEOX, MLA_ROPE_INTERLEAVED = 0, 1

EXPORTS = ("mla_default_scale", "mla_absorb_q", "mla_decode_workspace_size",
           "mla_decode_resolve_splits", "mla_decode_attention", "mla_decompress_v",
           "mla_decode_status", "mla_status_string", "mla_cache_append", "mla_prefill_workspace_size",
           "mla_prefill_attention", "mla_decode_attention_dcp", "mla_lse_combine", "mla_prolog_workspace_size",
           "mla_prolog", "mla_decode_attention_noalloc")


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_text(status)})")
        self.status = status


class mla_dims(ctypes.Structure):
    _fields_ = [("n_head", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("kv_rank", ctypes.c_int32)]


DimsLike = Union[mla_dims, Sequence[int], object]

_LIB = None


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python -m mla_latent_cache_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz, f32, vp = (ctypes.POINTER(mla_dims), ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p)
    L.mla_default_scale.restype = f32
    L.mla_default_scale.argtypes = [P]
    L.mla_absorb_q.restype = ctypes.c_int
    L.mla_absorb_q.argtypes = [P, i64, vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp]
    L.mla_decode_workspace_size.restype = ctypes.c_int
    L.mla_decode_workspace_size.argtypes = [P, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.mla_decode_resolve_splits.restype = i32
    L.mla_decode_resolve_splits.argtypes = [P, i32, i32, i32, i32]
    L.mla_decode_attention.restype = ctypes.c_int
    L.mla_decode_attention.argtypes = [P, f32, i32, i32, vp, vp, ctypes.c_int, i64, i32, vp, i32, vp,
                                       vp, ctypes.c_int, vp, vp, sz, i32, vp]
    L.mla_decode_attention_noalloc.restype = ctypes.c_int
    L.mla_decode_attention_noalloc.argtypes = [P, f32, i32, i32, vp, vp, ctypes.c_int, i64, i32, vp, i32, vp,
                                               vp, ctypes.c_int, vp, i32, vp]
    L.mla_decode_attention_dcp.restype = ctypes.c_int
    L.mla_decode_attention_dcp.argtypes = [P, f32, i32, i32, vp, vp, ctypes.c_int, i64, i32, vp, i32, vp,
                                           i32, i32, i32, vp, ctypes.c_int, vp, vp, sz, i32, vp]
    L.mla_lse_combine.restype = ctypes.c_int
    L.mla_lse_combine.argtypes = [i32, i64, i32, vp, vp, vp, ctypes.c_int, vp, vp]
    L.mla_prolog_workspace_size.restype = ctypes.c_int
    L.mla_prolog_workspace_size.argtypes = [P, ctypes.POINTER(mla_prolog_dims), i64, ctypes.POINTER(sz)]
    L.mla_prolog.restype = ctypes.c_int
    L.mla_prolog.argtypes = [P, ctypes.POINTER(mla_prolog_dims), i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                             ctypes.c_int, f32, f32, vp, ctypes.c_double, i32, vp, vp, ctypes.c_int, i64, i32, vp,
                             ctypes.c_int, vp, vp, sz, vp]
    L.mla_decompress_v.restype = ctypes.c_int
    L.mla_decompress_v.argtypes = [P, i64, vp, ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_int, vp]
    L.mla_decode_status.restype = ctypes.c_int
    L.mla_decode_status.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
    L.mla_cache_append.restype = ctypes.c_int
    L.mla_cache_append.argtypes = [P, i64, vp, vp, vp, ctypes.c_int, f32, vp, ctypes.c_double, i32, vp, vp,
                                   vp, ctypes.c_int, i64, i32, vp, vp]
    L.mla_prefill_workspace_size.restype = ctypes.c_int
    L.mla_prefill_workspace_size.argtypes = [P, i32, i32, i32, ctypes.POINTER(sz)]
    L.mla_prefill_attention.restype = ctypes.c_int
    L.mla_prefill_attention.argtypes = [P, f32, i32, i32, vp, vp, vp, vp, vp, ctypes.c_int, i64, i32, vp, i32, vp,
                                        vp, ctypes.c_int, vp, vp, sz, vp]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_status_string.argtypes = [ctypes.c_int]
    _LIB = L
    return L


def status_text(code: int) -> str:
    try:
        return lib().mla_status_string(int(code)).decode()
    except Exception:  # library missing: still give a readable message
        return "unknown"


def as_dims(d: DimsLike) -> mla_dims:
    if isinstance(d, mla_dims):
        return d
    if isinstance(d, (tuple, list)):
        return mla_dims(*[int(x) for x in d])
    return mla_dims(int(d.n_head), int(d.d_nope), int(d.d_rope), int(d.d_v), int(d.kv_rank))


def _check(fn: str, st: int) -> None:
    if st != MLA_OK:
        raise MlaError(fn, st)


def _dt(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    raise TypeError(f"unsupported tensor dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the MLA library must be device tensors")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MLA library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def mla_default_scale(dims: DimsLike) -> float:
    d = as_dims(dims)
    return float(lib().mla_default_scale(ctypes.byref(d)))


def mla_absorb_q(dims: DimsLike, q_nope, q_pe, w_uk, q_abs, stream=None) -> None:
    """q_abs[n][h] = [W_UK[h]^T q_nope[n][h] | q_pe[n][h]]; shapes as in include/mla.h."""
    d = as_dims(dims)
    n_tok = q_nope.numel() // max(1, d.n_head * d.d_nope)
    pe = q_pe if (q_pe is not None and q_pe.numel() > 0) else None
    _check("mla_absorb_q", lib().mla_absorb_q(ctypes.byref(d), n_tok, _ptr(q_nope), _ptr(pe), _ptr(w_uk),
                                               _dt(q_nope), _ptr(q_abs), _dt(q_abs), _stream(stream)))


def mla_decode_workspace_size(dims: DimsLike, batch: int, t_q: int, max_blocks: int,
                              block_size: int = 16, num_splits: int = 0) -> int:
    d = as_dims(dims)
    out = ctypes.c_size_t(0)
    _check("mla_decode_workspace_size",
           lib().mla_decode_workspace_size(ctypes.byref(d), batch, t_q, max_blocks, block_size, num_splits,
                                           ctypes.byref(out)))
    return int(out.value)


def mla_decode_resolve_splits(dims: DimsLike, batch: int, t_q: int, max_blocks: int,
                              num_splits: int = 0) -> int:
    d = as_dims(dims)
    return int(lib().mla_decode_resolve_splits(ctypes.byref(d), batch, t_q, max_blocks, num_splits))


def mla_decode_attention(dims: DimsLike, scale: float, q_abs, kv_cache, block_table, seq_lens, out_lat,
                         lse=None, workspace=None, num_splits: int = 0, stream=None) -> None:
    """Paged split-KV decode attention.  q_abs [B][t_q][H][D], kv_cache
    [num_blocks][16][D], block_table int32 [B][max_blocks], seq_lens int32 [B],
    out_lat [B][t_q][H][kv_rank], lse float32 [B][t_q][H] or None, workspace a
    uint8 device tensor of at least mla_decode_workspace_size() bytes."""
    d = as_dims(dims)
    B, t_q = int(q_abs.shape[0]), int(q_abs.shape[1])
    if workspace is None:
        raise ValueError("mla_decode_attention needs a workspace tensor")
    _check("mla_decode_attention", lib().mla_decode_attention(
        ctypes.byref(d), float(scale), B, t_q, _ptr(q_abs), _ptr(kv_cache), _dt(kv_cache),
        int(kv_cache.shape[0]), int(kv_cache.shape[1]), _ptr(block_table), int(block_table.shape[1]),
        _ptr(seq_lens), _ptr(out_lat), _dt(out_lat), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), int(num_splits), _stream(stream)))


def mla_decode_attention_noalloc(dims: DimsLike, scale: float, q_abs, kv_cache, block_table, seq_lens, out_lat,
                                 lse=None, num_splits: int = 0, stream=None) -> None:
    """mla_decode_attention with the library's own device scratch as the
    workspace (no allocation; calls that overlap on one GPU race)."""
    d = as_dims(dims)
    B, t_q = int(q_abs.shape[0]), int(q_abs.shape[1])
    _check("mla_decode_attention_noalloc", lib().mla_decode_attention_noalloc(
        ctypes.byref(d), float(scale), B, t_q, _ptr(q_abs), _ptr(kv_cache), _dt(kv_cache),
        int(kv_cache.shape[0]), int(kv_cache.shape[1]), _ptr(block_table), int(block_table.shape[1]),
        _ptr(seq_lens), _ptr(out_lat), _dt(out_lat), _ptr(lse), int(num_splits), _stream(stream)))


def mla_decode_attention_dcp(dims: DimsLike, scale: float, q_abs, kv_cache, block_table, seq_lens, dcp_world: int,
                             dcp_rank: int, dcp_interleave: int, out_lat, lse, workspace, num_splits: int = 0,
                             stream=None) -> None:
    """One rank's share of decode context parallelism: kv_cache / block_table
    hold the rank's rows only, seq_lens are the global lengths; out_lat and
    lse (required) receive the rank's partial result."""
    d = as_dims(dims)
    B, t_q = int(q_abs.shape[0]), int(q_abs.shape[1])
    if workspace is None:
        raise ValueError("mla_decode_attention_dcp needs a workspace tensor")
    _check("mla_decode_attention_dcp", lib().mla_decode_attention_dcp(
        ctypes.byref(d), float(scale), B, t_q, _ptr(q_abs), _ptr(kv_cache), _dt(kv_cache),
        int(kv_cache.shape[0]), int(kv_cache.shape[1]), _ptr(block_table), int(block_table.shape[1]),
        _ptr(seq_lens), int(dcp_world), int(dcp_rank), int(dcp_interleave), _ptr(out_lat), _dt(out_lat), _ptr(lse),
        _ptr(workspace), workspace.numel() * workspace.element_size(), int(num_splits), _stream(stream)))


def mla_lse_combine(o_parts, lse_parts, out, lse_out=None, stream=None) -> None:
    """Combine partial results: o_parts float32 [P][n][width], lse_parts
    float32 [P][n], out [n][width] (f32 or bf16), lse_out float32 [n] or None."""
    P = int(lse_parts.shape[0])
    n = lse_parts.numel() // max(1, P)
    width = o_parts.numel() // max(1, P * n)
    _check("mla_lse_combine", lib().mla_lse_combine(int(width), int(n), P, _ptr(o_parts), _ptr(lse_parts), _ptr(out),
                                                    _dt(out), _ptr(lse_out), _stream(stream)))


class mla_prolog_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("q_rank", ctypes.c_int32)]


def mla_prolog_workspace_size(dims: DimsLike, hidden: int, q_rank: int, n_tok: int) -> int:
    d = as_dims(dims)
    pd = mla_prolog_dims(hidden, q_rank)
    out = ctypes.c_size_t(0)
    _check("mla_prolog_workspace_size", lib().mla_prolog_workspace_size(ctypes.byref(d), ctypes.byref(pd), int(n_tok),
                                                                        ctypes.byref(out)))
    return int(out.value)


def mla_prolog(dims: DimsLike, x, w_dq, w_uq, w_qr, w_uk, w_dkv, w_kr, gamma_q, gamma_kv, eps_q: float, eps_kv: float,
               positions, rope_base: float, rope_style: int, slot_mapping, kv_cache, q_abs, workspace, data_err=None,
               stream=None) -> None:
    """Fused prolog: x [n_tok][hidden] and the [out][in] projection weights
    -> q_abs [n_tok][H][kv_rank + d_rope] and the cache rows slot_mapping[n]."""
    d = as_dims(dims)
    n_tok, hidden = int(x.shape[0]), int(x.shape[1])
    pd = mla_prolog_dims(hidden, int(w_dq.shape[0]))
    _check("mla_prolog", lib().mla_prolog(
        ctypes.byref(d), ctypes.byref(pd), n_tok, _ptr(x), _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), _ptr(w_uk), _ptr(w_dkv),
        _ptr(w_kr), _ptr(gamma_q), _ptr(gamma_kv), _dt(x), float(eps_q), float(eps_kv), _ptr(positions),
        float(rope_base), int(rope_style), _ptr(slot_mapping), _ptr(kv_cache), _dt(kv_cache), int(kv_cache.shape[0]),
        int(kv_cache.shape[1]), _ptr(q_abs), _dt(q_abs), _ptr(data_err), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_decompress_v(dims: DimsLike, o_lat, w_uv, out, stream=None) -> None:
    """out[n][h][j] = sum_l W_UV[h][j][l] o_lat[n][h][l]."""
    d = as_dims(dims)
    n_tok = o_lat.numel() // max(1, d.n_head * d.kv_rank)
    _check("mla_decompress_v", lib().mla_decompress_v(ctypes.byref(d), n_tok, _ptr(o_lat), _dt(o_lat),
                                                       _ptr(w_uv), _dt(w_uv), _ptr(out), _dt(out),
                                                       _stream(stream)))


def mla_decode_status(workspace, stream=None) -> int:
    """MLA_DATA_* bits recorded by the last decode on this workspace (waits for the stream)."""
    flags = ctypes.c_uint32(0)
    _check("mla_decode_status", lib().mla_decode_status(_ptr(workspace), ctypes.byref(flags), _stream(stream)))
    return int(flags.value)


def mla_cache_append(dims: DimsLike, c_kv, k_pe, gamma, eps: float, positions, rope_base: float,
                     rope_style: int, q_pe, slot_mapping, kv_cache, data_err=None, stream=None) -> None:
    """Cache-append prolog: kv_cache row slot_mapping[n] <- [RmsNorm(c_kv[n]) |
    rope(k_pe[n], positions[n])], q_pe rotated in place.  c_kv [n_tok][kv_rank],
    k_pe [n_tok][d_rope], gamma [kv_rank] or None, positions int32 [n_tok],
    q_pe [n_tok][H][d_rope] or None, slot_mapping int64 [n_tok], kv_cache
    [num_blocks][16][D], data_err int32 [1] device tensor or None."""
    d = as_dims(dims)
    n_tok = c_kv.numel() // max(1, d.kv_rank)
    pe = k_pe if (k_pe is not None and k_pe.numel() > 0) else None
    qpe = q_pe if (q_pe is not None and q_pe.numel() > 0) else None
    _check("mla_cache_append", lib().mla_cache_append(
        ctypes.byref(d), n_tok, _ptr(c_kv), _ptr(pe), _ptr(gamma), _dt(c_kv), float(eps), _ptr(positions),
        float(rope_base), int(rope_style), _ptr(qpe), _ptr(slot_mapping), _ptr(kv_cache), _dt(kv_cache),
        int(kv_cache.shape[0]), int(kv_cache.shape[1]), _ptr(data_err), _stream(stream)))


def mla_prefill_workspace_size(dims: DimsLike, batch: int, max_blocks: int, block_size: int = 16) -> int:
    d = as_dims(dims)
    out = ctypes.c_size_t(0)
    _check("mla_prefill_workspace_size",
           lib().mla_prefill_workspace_size(ctypes.byref(d), batch, max_blocks, block_size, ctypes.byref(out)))
    return int(out.value)


def mla_prefill_attention(dims: DimsLike, scale: float, q_nope, q_pe, w_uk, w_uv, kv_cache, block_table, seq_lens,
                          out, lse=None, workspace=None, stream=None) -> None:
    """Naive-form prefill attention.  q_nope [B][t_q][H][d_nope], q_pe
    [B][t_q][H][d_rope] or None, w_uk [H][d_nope][kv_rank], w_uv
    [H][d_v][kv_rank], kv_cache [num_blocks][16][D], block_table int32
    [B][max_blocks], seq_lens int32 [B], out [B][t_q][H][d_v], lse float32
    [B][t_q][H] or None, workspace a uint8 device tensor of at least
    mla_prefill_workspace_size() bytes."""
    d = as_dims(dims)
    B, t_q = int(q_nope.shape[0]), int(q_nope.shape[1])
    if workspace is None:
        raise ValueError("mla_prefill_attention needs a workspace tensor")
    pe = q_pe if (q_pe is not None and q_pe.numel() > 0) else None
    _check("mla_prefill_attention", lib().mla_prefill_attention(
        ctypes.byref(d), float(scale), B, t_q, _ptr(q_nope), _ptr(pe), _ptr(w_uk), _ptr(w_uv), _ptr(kv_cache),
        _dt(kv_cache), int(kv_cache.shape[0]), int(kv_cache.shape[1]), _ptr(block_table),
        int(block_table.shape[1]), _ptr(seq_lens), _ptr(out), _dt(out), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_status_string(code: int) -> str:
    return lib().mla_status_string(int(code)).decode()
