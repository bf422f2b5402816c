"""CPU oracle for MLA latent-cache decode -- TEST INFRASTRUCTURE ONLY.

Plain C (``mla_oracle.c``), float64 arithmetic, loaded through ctypes.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``mla_latent_cache_amd``) and never imports it.

Inputs are numpy arrays stored as float32, bfloat16 bit patterns (uint16) or
float64; outputs are float64.  Every function is pinned by the ``not gpu``
tests in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

F32, BF16, F64 = 0, 1, 2


def _load():
    global _LIB
    if _LIB is not None:
        return _LIB
    path = os.environ.get("MLA_ORACLE_LIB") or _build.library_path()
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    i32, i64, dbl, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.mla_oracle_threads.restype = i32
    lib.mla_oracle_set_threads.argtypes = [i32]
    lib.mla_oracle_scale.restype = dbl
    lib.mla_oracle_scale.argtypes = [i32, i32]
    lib.mla_oracle_absorb.argtypes = [i32, i32, i32, i32, i64, vp, vp, i32, vp, i32, vp]
    lib.mla_oracle_decompress.argtypes = [i32, i32, i32, i64, vp, i32, vp, i32, vp]
    lib.mla_oracle_decode.restype = i64
    lib.mla_oracle_decode.argtypes = [i32, i32, i32, i32, i32, i32, vp, i32, vp, i32, i64, i32,
                                      vp, i32, vp, dbl, vp, i64, vp, vp]
    lib.mla_oracle_decode_share.restype = i64
    lib.mla_oracle_decode_share.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, i32, vp, i32, i64,
                                            i32, vp, i32, vp, dbl, vp, i64, vp, vp]
    lib.mla_oracle_attend_absorbed.restype = i64
    lib.mla_oracle_attend_absorbed.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, i32,
                                               vp, vp, i32, vp, i32, i64, i32, vp, i32, vp, dbl,
                                               vp, i64, vp, vp, vp]
    lib.mla_oracle_attend_naive.restype = i64
    lib.mla_oracle_attend_naive.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, i32, vp,
                                            vp, i32, vp, i32, i64, i32, vp, i32, vp, dbl, vp,
                                            i64, vp, vp]
    lib.mla_oracle_rope_interleaved.argtypes = [vp, i32, dbl, dbl]
    lib.mla_oracle_rope_neox.argtypes = [vp, i32, dbl, dbl]
    lib.mla_oracle_norm_to_neox_perm.argtypes = [i32, vp]
    lib.mla_oracle_rmsnorm.argtypes = [vp, i32, i64, i32, vp, i32, dbl, vp]
    lib.mla_oracle_rope_rows.argtypes = [vp, i32, i64, i32, i32, vp, dbl, i32, vp]
    lib.mla_oracle_cache_append.restype = i64
    lib.mla_oracle_cache_append.argtypes = [i32, i32, i64, vp, vp, i32, vp, i32, dbl, vp, dbl,
                                            i32, vp, vp, i64]
    _LIB = lib
    return lib


def _code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle input must be float32, bf16 bits (uint16) or float64, got {a.dtype}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return _load().mla_oracle_threads()


def set_threads(n: int) -> None:
    _load().mla_oracle_set_threads(int(n))


def scale(d_nope: int, d_rope: int) -> float:
    """Softmax scale 1/sqrt(d_nope + d_rope) (memra mla.rs page, MlaDims::scale)."""
    return _load().mla_oracle_scale(int(d_nope), int(d_rope))


@dataclass
class Dims:
    n_head: int
    d_nope: int
    d_rope: int
    d_v: int
    kv_rank: int


def absorb(dims: Dims, q_nope, q_pe, w_uk) -> np.ndarray:
    """q_abs[n][h] = [W_UK[h]^T q_nope[n][h] | q_pe[n][h]], shape [n_tok][H][kv_rank+d_rope]."""
    q_nope, q_pe, w_uk = _c(q_nope), _c(q_pe), _c(w_uk)
    n_tok = q_nope.size // (dims.n_head * dims.d_nope)
    out = np.empty((n_tok, dims.n_head, dims.kv_rank + dims.d_rope), np.float64)
    if q_pe.size == 0:
        q_pe = np.zeros(1, q_nope.dtype)
    _load().mla_oracle_absorb(dims.n_head, dims.d_nope, dims.d_rope, dims.kv_rank, n_tok,
                              _p(q_nope), _p(q_pe), _code(q_nope), _p(w_uk), _code(w_uk), _p(out))
    return out


def decompress(dims: Dims, o_lat, w_uv) -> np.ndarray:
    """out[n][h][j] = sum_l W_UV[h][j][l] o_lat[n][h][l], shape [n_tok][H][d_v]."""
    o_lat, w_uv = _c(o_lat), _c(w_uv)
    n_tok = o_lat.size // (dims.n_head * dims.kv_rank)
    out = np.empty((n_tok, dims.n_head, dims.d_v), np.float64)
    _load().mla_oracle_decompress(dims.n_head, dims.d_v, dims.kv_rank, n_tok, _p(o_lat),
                                  _code(o_lat), _p(w_uv), _code(w_uv), _p(out))
    return out


@dataclass
class Paged:
    """A paged latent cache: kv [num_blocks][block_size][kv_rank+d_rope]."""
    kv: np.ndarray
    block_table: np.ndarray  # int32 [B][max_blocks]
    seq_lens: np.ndarray     # int32 [B]
    block_size: int = 16

    @property
    def num_blocks(self) -> int:
        return self.kv.shape[0]

    @property
    def batch(self) -> int:
        return self.seq_lens.shape[0]

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]


def _sel(sel):
    if sel is None:
        return None, 0
    s = np.ascontiguousarray(np.asarray(sel, dtype=np.int32).reshape(-1, 3))
    return s, s.shape[0]


def decode(dims: Dims, t_q: int, q_abs, cache: Paged, scale_: float, sel=None,
           method: str = "twopass"):
    """Attention of absorbed queries q_abs [B][t_q][H][D] over the paged cache.

    method "twopass" is the plain softmax definition; "online" is the
    single-pass running-max recurrence.  Returns (o_lat [n][kv_rank],
    lse [n], n_invalid) for the selected (b, i, h) items (all when sel is None,
    in row-major (b, i, h) order).
    """
    q_abs = _c(q_abs)
    kv = _c(cache.kv)
    bt = _c(cache.block_table.astype(np.int32, copy=False))
    sl = _c(cache.seq_lens.astype(np.int32, copy=False))
    s, n_sel = _sel(sel)
    n = n_sel if s is not None else cache.batch * t_q * dims.n_head
    o = np.empty((n, dims.kv_rank), np.float64)
    lse = np.empty(n, np.float64)
    bad = _load().mla_oracle_decode(0 if method == "twopass" else 1, dims.n_head, dims.kv_rank,
                                    dims.d_rope, cache.batch, t_q, _p(q_abs), _code(q_abs),
                                    _p(kv), _code(kv), cache.num_blocks, cache.block_size,
                                    _p(bt), cache.max_blocks, _p(sl), float(scale_), _p(s), n_sel,
                                    _p(o), _p(lse))
    return o, lse, int(bad)


def decode_share(dims: Dims, t_q: int, q_abs, cache: Paged, scale_: float, world: int, rank: int,
                 interleave: int = 1, sel=None):
    """One rank's share of decode context parallelism (two-pass attention over
    the visible rows j with (j // interleave) % world == rank of the request's
    whole paged cache).  Returns (o_lat [n][kv_rank], lse [n], n_invalid)."""
    if not (world >= 1 and 0 <= rank < world and interleave >= 1):
        raise ValueError("need world >= 1, 0 <= rank < world, interleave >= 1")
    q_abs = _c(q_abs)
    kv = _c(cache.kv)
    bt = _c(cache.block_table.astype(np.int32, copy=False))
    sl = _c(cache.seq_lens.astype(np.int32, copy=False))
    s, n_sel = _sel(sel)
    n = n_sel if s is not None else cache.batch * t_q * dims.n_head
    o = np.empty((n, dims.kv_rank), np.float64)
    lse = np.empty(n, np.float64)
    bad = _load().mla_oracle_decode_share(int(world), int(rank), int(interleave), dims.n_head, dims.kv_rank,
                                          dims.d_rope, cache.batch, t_q, _p(q_abs), _code(q_abs), _p(kv),
                                          _code(kv), cache.num_blocks, cache.block_size, _p(bt),
                                          cache.max_blocks, _p(sl), float(scale_), _p(s), n_sel, _p(o),
                                          _p(lse))
    return o, lse, int(bad)


def lse_combine(o_parts, lse_parts):
    """Combine partial attention results over disjoint row sets (the split
    merge): with M = max_p lse_p and w_p = exp(lse_p - M),
    o = sum_p w_p o_p / sum_p w_p and lse = M + ln sum_p w_p; parts with
    lse = -inf carry no weight (their o is not read); all -inf gives zeros and
    -inf; a NaN LSE in any part gives NaN.  o_parts [P][n][R], lse_parts
    [P][n]; float64 results ([n][R], [n])."""
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    P, n = lse_parts.shape
    o = np.zeros((n, o_parts.shape[2]), np.float64)
    lse = np.full(n, -np.inf)
    for k in range(n):
        ls = lse_parts[:, k]
        if np.isnan(ls).any():
            o[k] = np.nan
            lse[k] = np.nan
            continue
        M = ls.max()
        if M == -np.inf:
            continue
        acc = np.zeros(o_parts.shape[2], np.float64)
        wsum = 0.0
        for p in range(P):
            if ls[p] == -np.inf:
                continue
            wp = np.exp(ls[p] - M)
            acc += wp * o_parts[p, k]
            wsum += wp
        o[k] = acc / wsum
        lse[k] = M + np.log(wsum)
    return o, lse


def _full_args(dims, t_q, q_nope, q_pe, w_uk, w_uv, cache):
    q_nope, w_uk, w_uv = _c(q_nope), _c(w_uk), _c(w_uv)
    q_pe = _c(q_pe) if q_pe is not None and q_pe.size else np.zeros(1, q_nope.dtype)
    kv = _c(cache.kv)
    bt = _c(cache.block_table.astype(np.int32, copy=False))
    sl = _c(cache.seq_lens.astype(np.int32, copy=False))
    if _code(w_uk) != _code(w_uv):
        raise TypeError("w_uk and w_uv must share a storage type")
    return q_nope, q_pe, w_uk, w_uv, kv, bt, sl


def attend_absorbed(dims: Dims, t_q: int, q_nope, q_pe, w_uk, w_uv, cache: Paged,
                    scale_: float, sel=None):
    """Full absorbed form: absorb, latent attention, decompress.

    Returns (out [n][d_v], o_lat [n][kv_rank], lse [n], n_invalid).
    """
    q_nope, q_pe, w_uk, w_uv, kv, bt, sl = _full_args(dims, t_q, q_nope, q_pe, w_uk, w_uv, cache)
    s, n_sel = _sel(sel)
    n = n_sel if s is not None else cache.batch * t_q * dims.n_head
    out = np.empty((n, dims.d_v), np.float64)
    o = np.empty((n, dims.kv_rank), np.float64)
    lse = np.empty(n, np.float64)
    bad = _load().mla_oracle_attend_absorbed(
        dims.n_head, dims.d_nope, dims.d_rope, dims.d_v, dims.kv_rank, cache.batch, t_q,
        _p(q_nope), _p(q_pe), _code(q_nope), _p(w_uk), _p(w_uv), _code(w_uk), _p(kv), _code(kv),
        cache.num_blocks, cache.block_size, _p(bt), cache.max_blocks, _p(sl), float(scale_),
        _p(s), n_sel, _p(out), _p(o), _p(lse))
    return out, o, lse, int(bad)


def attend_naive(dims: Dims, t_q: int, q_nope, q_pe, w_uk, w_uv, cache: Paged,
                 scale_: float, sel=None):
    """Naive form: per-head decompression of the cache, attention at width
    d_nope + d_rope.  Returns (out [n][d_v], lse [n], n_invalid)."""
    q_nope, q_pe, w_uk, w_uv, kv, bt, sl = _full_args(dims, t_q, q_nope, q_pe, w_uk, w_uv, cache)
    s, n_sel = _sel(sel)
    n = n_sel if s is not None else cache.batch * t_q * dims.n_head
    out = np.empty((n, dims.d_v), np.float64)
    lse = np.empty(n, np.float64)
    bad = _load().mla_oracle_attend_naive(
        dims.n_head, dims.d_nope, dims.d_rope, dims.d_v, dims.kv_rank, cache.batch, t_q,
        _p(q_nope), _p(q_pe), _code(q_nope), _p(w_uk), _p(w_uv), _code(w_uk), _p(kv), _code(kv),
        cache.num_blocks, cache.block_size, _p(bt), cache.max_blocks, _p(sl), float(scale_),
        _p(s), n_sel, _p(out), _p(lse))
    return out, lse, int(bad)


def rope_interleaved(x, pos: float, base: float) -> np.ndarray:
    """Interleaved ("NORM") RoPE over all of x (float64 copy returned)."""
    y = np.array(x, dtype=np.float64, copy=True)
    _load().mla_oracle_rope_interleaved(_p(y), y.size, float(pos), float(base))
    return y


def rope_neox(x, pos: float, base: float) -> np.ndarray:
    """NEOX RoPE over all of x (float64 copy returned)."""
    y = np.array(x, dtype=np.float64, copy=True)
    _load().mla_oracle_rope_neox(_p(y), y.size, float(pos), float(base))
    return y


def norm_to_neox_perm(n_dims: int) -> np.ndarray:
    """Interleaved index -> NEOX index permutation."""
    p = np.empty(n_dims, np.int32)
    _load().mla_oracle_norm_to_neox_perm(int(n_dims), _p(p))
    return p


NEOX, INTERLEAVED = 0, 1


def rmsnorm(x, gamma=None, eps: float = 0.0) -> np.ndarray:
    """RmsNorm of every row of x [..., width] (CANN aclnnMlaProlog, RmsNorm
    formula): gamma * x / sqrt(mean(x^2) + eps).  float64 result."""
    x = _c(x)
    width = x.shape[-1]
    n_rows = x.size // width if width else 0
    y = np.empty(x.shape, np.float64)
    g = None if gamma is None else _c(gamma)
    _load().mla_oracle_rmsnorm(_p(x), _code(x), n_rows, width, _p(g), 0 if g is None else _code(g),
                               float(eps), _p(y))
    return y


def rope_rows(x, positions, base: float, style: int = NEOX) -> np.ndarray:
    """RoPE of x [n_rows][n_heads][n_dims], every head of row r at position
    positions[r] (mla.rs rope_neox / rope_interleaved).  float64 result."""
    x = _c(x)
    n_rows, n_heads, n_dims = x.shape
    pos = _c(np.asarray(positions, dtype=np.int32))
    assert pos.shape == (n_rows,)
    y = np.empty(x.shape, np.float64)
    _load().mla_oracle_rope_rows(_p(x), _code(x), n_rows, n_heads, n_dims, _p(pos), float(base),
                                 int(style), _p(y))
    return y


def cache_append(cache_rows, kv_rank: int, c_kv, k_pe, gamma, eps: float, positions,
                 base: float, style: int, slots):
    """Cache-append prolog (vLLM cpu_mla do_kv_cache_update, fed by the
    aclnnMlaProlog c^KV = RmsNorm(.) and k^R = ROPE(.) formulas).

    cache_rows: float64 [num_slots][kv_rank + d_rope], updated in place.  Row
    slots[n] becomes [RmsNorm(c_kv[n]) | rope(k_pe[n], positions[n])];
    negative slots are skipped, slots >= num_slots are skipped and counted.
    Returns the count of out-of-range slots.
    """
    assert cache_rows.dtype == np.float64 and cache_rows.flags.c_contiguous
    num_slots, width = cache_rows.shape
    d_rope = width - kv_rank
    c_kv = _c(c_kv)
    n_tok = c_kv.size // kv_rank
    k_pe = _c(k_pe) if d_rope else np.zeros(1, c_kv.dtype)
    pos = _c(np.asarray(positions, dtype=np.int32)) if d_rope else np.zeros(max(n_tok, 1), np.int32)
    sl = _c(np.asarray(slots, dtype=np.int64))
    assert sl.shape == (n_tok,)
    g = None if gamma is None else _c(gamma)
    bad = _load().mla_oracle_cache_append(
        kv_rank, d_rope, n_tok, _p(c_kv), _p(k_pe), _code(c_kv), _p(g),
        0 if g is None else _code(g), float(eps), _p(pos), float(base), int(style), _p(sl),
        _p(cache_rows), num_slots)
    return int(bad)


def prolog(dims: Dims, x, w_dq, w_uq, w_qr, w_uk, w_dkv, w_kr, gamma_q, gamma_kv, eps_q: float, eps_kv: float,
           positions, base: float, style: int, slots, cache_rows):
    """The fused MLA prolog (CANN aclnnMlaProlog, its four paths), in the
    order the page's formulas give, float64 throughout:
        c^Q  = RmsNorm(x W^DQ)             (gamma_q, eps_q)
        q^C  = c^Q W^UQ,  q^N = q^C W^UK   (per head; W^UK is the absorb step's)
        q^R  = ROPE(c^Q W^QR)              (each token at its position)
        c^KV = RmsNorm(x W^DKV), k^R = ROPE(x W^KR), both written to cache
               row slots[n] (the cache append: gamma_kv, eps_kv)
    Weights are stored [out][in]: w_dq [q_rank][hidden], w_dkv
    [kv_rank][hidden], w_kr [d_rope][hidden], w_uq [H d_nope][q_rank] and
    w_qr [H d_rope][q_rank] (output feature h * width + j); w_uk
    [H][d_nope][kv_rank].  x [n][hidden].  cache_rows float64
    [num_slots][kv_rank + d_rope] is updated in place.  Returns
    (q_abs [n][H][kv_rank + d_rope] = [q^N | q^R], out-of-range slot count).
    """
    H, dn, dr, R = dims.n_head, dims.d_nope, dims.d_rope, dims.kv_rank
    x = np.asarray(_widen(x), np.float64)
    n = x.shape[0]
    cq = rmsnorm(x @ np.asarray(_widen(w_dq), np.float64).T, gamma_q, eps_q)
    qc = (cq @ np.asarray(_widen(w_uq), np.float64).T).reshape(n, H, dn)
    qr = np.zeros((n, H, 0), np.float64)
    if dr:
        qr = rope_rows((cq @ np.asarray(_widen(w_qr), np.float64).T).reshape(n, H, dr), positions, base, style)
    q_abs = absorb(dims, qc, qr, w_uk).reshape(n, H, R + dr)
    ckv = x @ np.asarray(_widen(w_dkv), np.float64).T
    kr = x @ np.asarray(_widen(w_kr), np.float64).T if dr else None
    bad = cache_append(cache_rows, R, ckv, kr, gamma_kv, eps_kv, positions, base, style, slots)
    return q_abs, bad


def _widen(a):
    """Stored values as float64 (bfloat16 bit patterns widened exactly)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
