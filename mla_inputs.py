"""Seeded synthetic inputs for MLA latent-cache decode.

The one module that both the HIP path's tests/benchmark and the oracle's
tests draw inputs from.  It holds none of the method's arithmetic: it only
draws random numbers, rounds them to a storage type, shapes the synthetic
latent rows to unit RMS (the pages state the cache holds already-normalised
c_kv rows), and lays rows out in a paged cache.

Random numbers
--------------
Counter-based SplitMix64 (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014): output k of a stream with key
K is mix(K + (k + 1) * 0x9E3779B97F4A7C15), where mix is the SplitMix64
finaliser.  Each tensor has its own key, derived from (config seed, tensor
tag).  Normals come from the Box-Muller transform (1958), one 64-bit draw per
pair: the high 32 bits give u1, the low 32 bits give u2.

Cache rows are indexed by their logical position (request, row), never by
the physical block they land in, so a relabelled block table holds exactly
the same values.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

BLOCK_SIZE = 16
SPARE_BLOCKS = 64
RMS_EPS = 1e-6
BF16_QNAN = np.uint16(0x7FC0)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------
# SplitMix64
# --------------------------------------------------------------------------
def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def draws(key: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the stream with this key (uint64)."""
    k = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + k * GOLDEN)


def _fnv1a64(s: str) -> int:
    h = 0xCBF29CE484222325
    for ch in s.encode():
        h ^= ch
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def tensor_key(seed: int, tag: str) -> int:
    """Stream key for one tensor of one configuration."""
    return int(mix64(np.array([(seed * 0x2545F4914F6CDD1D ^ _fnv1a64(tag)) & 0xFFFFFFFFFFFFFFFF],
                              dtype=np.uint64))[0])


def normals(key: int, start: int, count: int) -> np.ndarray:
    """Standard normals start .. start+count-1 of a stream (float64).

    Pair k = draw k: u1 = (hi32 + 0.5) / 2^32, u2 = (lo32 + 0.5) / 2^32,
    value 2k = r cos(2 pi u2), value 2k+1 = r sin(2 pi u2), r = sqrt(-2 ln u1).
    """
    if count <= 0:
        return np.zeros(0, np.float64)
    p0, p1 = start // 2, (start + count - 1) // 2 + 1
    z = draws(key, p0, p1 - p0)
    u1 = ((z >> np.uint64(32)).astype(np.float64) + 0.5) * (1.0 / 4294967296.0)
    u2 = ((z & np.uint64(0xFFFFFFFF)).astype(np.float64) + 0.5) * (1.0 / 4294967296.0)
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * (p1 - p0), np.float64)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    off = start - 2 * p0
    return out[off:off + count]


def normals_parallel(key: int, count: int, chunk: int = 1 << 20) -> np.ndarray:
    """normals(key, 0, count), computed in chunks on a thread pool (the
    stream is counter-based, so chunks are independent; identical values)."""
    out = np.empty(count, np.float64)
    starts = list(range(0, count, 2 * (chunk // 2)))

    def work(s0):
        n = min(2 * (chunk // 2), count - s0)
        out[s0:s0 + n] = normals(key, s0, n)

    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(work, starts))
    return out


def uniforms(key: int, start: int, count: int) -> np.ndarray:
    """Uniforms in [0, 1) from the top 53 bits of each draw (float64)."""
    z = draws(key, start, count)
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


# --------------------------------------------------------------------------
# Storage types
# --------------------------------------------------------------------------
def to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even);
    NaN stays a quiet NaN with its sign.  Returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    r = r.astype(np.uint16)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values -> storage array: float32, or bfloat16 bits (uint16)."""
    x32 = np.asarray(x, dtype=np.float32)
    return x32 if dtype == "f32" else to_bf16_bits(x32)


def store_parallel(x: np.ndarray, dtype: str, chunk: int = 1 << 20) -> np.ndarray:
    """store() of a flat array, in chunks on a thread pool (same values)."""
    x = np.ascontiguousarray(x).reshape(-1)
    out = np.empty(x.size, np.float32 if dtype == "f32" else np.uint16)

    def work(s0):
        out[s0:s0 + chunk] = store(x[s0:s0 + chunk], dtype)

    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(work, range(0, x.size, chunk)))
    return out


def widen(a: np.ndarray) -> np.ndarray:
    """Storage array -> float32 values."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


# --------------------------------------------------------------------------
# Configurations
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Spec:
    """One synthetic workload: geometry, lengths, distributions and seed."""
    name: str
    n_head: int
    d_nope: int
    d_rope: int
    d_v: int
    kv_rank: int
    dtype: str                  # "f32" or "bf16"
    batch: int
    t_q: int
    max_blocks: int
    seed: int
    lengths: str = "fixed"      # "fixed" or "ragged"
    seq_len: int = 0            # fixed length, or the ragged upper bound
    fixed_lens: tuple = ()      # explicit lengths (overrides seq_len)
    zero_requests: tuple = ()   # requests forced to length 0
    q_given: bool = False       # absorbed queries drawn directly (no W_UK/W_UV)
    value_scale: float = 1.0    # multiplier of every drawn tensor
    rms_norm_ckv: bool = True   # c_kv rows shaped to unit RMS
    weight_scale: Optional[float] = None  # default 1/sqrt(kv_rank)
    scale: Optional[float] = None         # softmax scale (default 1/sqrt(d_nope+d_rope))
    spare_blocks: int = SPARE_BLOCKS

    @property
    def D(self) -> int:
        return self.kv_rank + self.d_rope

    def softmax_scale(self) -> float:
        if self.scale is not None:
            return float(self.scale)
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)

    def wscale(self) -> float:
        if self.weight_scale is not None:
            return float(self.weight_scale)
        return 1.0 / math.sqrt(self.kv_rank)


SPECS = {
    # Tiny f32 decode: every tensor N(0,1) * 0.1, lengths {5, 37}.
    "tiny_f32": Spec("tiny_f32", 4, 16, 8, 16, 32, "f32", batch=2, t_q=1, max_blocks=3,
                     seed=101, fixed_lens=(5, 37), value_scale=0.1, rms_norm_ckv=False,
                     weight_scale=0.1, spare_blocks=2),
    # GLM-5.2 geometry decode: 64 heads, nope 192, rope 64, v 256, rank 512.
    "glm52_decode": Spec("glm52_decode", 64, 192, 64, 256, 512, "bf16", batch=32, t_q=1,
                         max_blocks=256, seed=202, seq_len=4096),
    # DeepSeek-V3-shaped ragged decode: 128 heads, 576-wide absorbed queries given directly,
    # lengths uniform in [0, 32768] with requests 0 and 63 empty.  Scale 1/sqrt(128+64).
    "dsv3_ragged": Spec("dsv3_ragged", 128, 128, 64, 0, 512, "bf16", batch=64, t_q=1,
                        max_blocks=2048, seed=303, lengths="ragged", seq_len=32768,
                        zero_requests=(0, 63), q_given=True),
    # Multi-token causal decode, t_q = 4 on GLM-5.2 dims.
    "glm52_causal_tq4": Spec("glm52_causal_tq4", 64, 192, 64, 256, 512, "bf16", batch=16, t_q=4,
                             max_blocks=512, seed=404, seq_len=8192),
    # NoPE geometry (d_rope 0): one long request, then many short ones.
    "nope_long": Spec("nope_long", 64, 256, 0, 256, 512, "bf16", batch=1, t_q=1,
                      max_blocks=8192, seed=505, seq_len=131072),
    "nope_wide": Spec("nope_wide", 64, 256, 0, 256, 512, "bf16", batch=256, t_q=1,
                      max_blocks=64, seed=506, seq_len=1024),
    # Chunked prefill on GLM-5.2 dims: 2 requests of 4096 rows whose last 1024
    # are the new (causal) queries.
    "glm52_prefill": Spec("glm52_prefill", 64, 192, 64, 256, 512, "bf16", batch=2, t_q=1024,
                          max_blocks=256, seed=606, seq_len=4096),
}


def seq_lens_for(spec: Spec) -> np.ndarray:
    if spec.fixed_lens:
        lens = np.array(spec.fixed_lens, dtype=np.int64)
    elif spec.lengths == "ragged":
        u = uniforms(tensor_key(spec.seed, "seq_lens"), 0, spec.batch)
        lens = np.floor(u * (spec.seq_len + 1)).astype(np.int64)
    else:
        lens = np.full(spec.batch, spec.seq_len, dtype=np.int64)
    for b in spec.zero_requests:
        lens[b] = 0
    return lens.astype(np.int32)


@dataclass
class Case:
    """Materialised inputs of one workload.  Storage arrays are float32 or
    bfloat16 bit patterns (uint16); shapes are row-major."""
    spec: Spec
    seq_lens: np.ndarray            # int32 [B]
    block_table: np.ndarray         # int32 [B][max_blocks], -1 where unused
    kv: np.ndarray                  # [num_blocks][16][D]
    q_nope: Optional[np.ndarray]    # [B*t_q][H][d_nope]
    q_pe: Optional[np.ndarray]      # [B*t_q][H][d_rope]
    w_uk: Optional[np.ndarray]      # [H][d_nope][kv_rank]
    w_uv: Optional[np.ndarray]      # [H][d_v][kv_rank]
    q_abs: Optional[np.ndarray]     # [B][t_q][H][D] (only when drawn directly)
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return self.kv.shape[0]

    @property
    def scale(self) -> float:
        return self.spec.softmax_scale()


def _draw(spec: Spec, tag: str, shape, scale: float) -> np.ndarray:
    n = int(np.prod(shape))
    x = normals(tensor_key(spec.seed, tag), 0, n) * scale
    return store(x.reshape(shape), spec.dtype)


def _poison(dtype: str):
    return np.float32(np.nan) if dtype == "f32" else BF16_QNAN


def block_permutation(key: int, num_blocks: int) -> np.ndarray:
    """A random permutation of the physical block ids (argsort of draws)."""
    return np.argsort(draws(key, 0, num_blocks), kind="stable").astype(np.int64)


def _rows(spec: Spec, g0: int, n: int) -> np.ndarray:
    """Cache rows g0 .. g0+n-1 in logical (request-major) order, float64,
    before rounding to the storage type: [c_kv | k_pe]."""
    Lk, R = spec.kv_rank, spec.d_rope
    c = normals(tensor_key(spec.seed, "c_kv"), g0 * Lk, n * Lk).reshape(n, Lk)
    if spec.rms_norm_ckv:
        c = c / np.sqrt(np.mean(c * c, axis=1, keepdims=True) + RMS_EPS)
    rows = np.empty((n, spec.D), np.float64)
    rows[:, :Lk] = c * spec.value_scale
    if R:
        rows[:, Lk:] = normals(tensor_key(spec.seed, "k_pe"), g0 * R, n * R).reshape(n, R) * spec.value_scale
    return rows


def logical_rows(spec: Spec, seq_lens, b: int) -> np.ndarray:
    """The stored rows of request b, in logical order, widened to float64.

    Drawn from the same streams as make_case but never through a block table,
    so a test can check paged gathers against it."""
    lens = np.maximum(np.asarray(seq_lens, dtype=np.int64), 0)
    g0 = int(lens[:b].sum())
    return widen(store(_rows(spec, g0, int(lens[b])), spec.dtype)).astype(np.float64)


def make_case(spec: Spec, seq_lens=None, relabel_seed: Optional[int] = None,
              poison: bool = True, threads: Optional[int] = None) -> Case:
    """Draw every input of a workload.

    seq_lens overrides the spec's lengths (the cache holds exactly the rows
    those lengths need).  relabel_seed draws a different block permutation
    with identical logical contents.  Spare blocks and the tail rows of each
    request's last block are NaN when poison is set.
    """
    lens = np.asarray(seq_lens_for(spec) if seq_lens is None else seq_lens, dtype=np.int64)
    B, D, R, Lk = spec.batch, spec.D, spec.d_rope, spec.kv_rank
    assert lens.shape == (B,)
    nblk = (np.maximum(lens, 0) + BLOCK_SIZE - 1) // BLOCK_SIZE
    assert int(nblk.max(initial=0)) <= spec.max_blocks, "a length exceeds the block table row"
    used = int(nblk.sum())
    num_blocks = used + spec.spare_blocks
    perm_key = tensor_key(spec.seed if relabel_seed is None else relabel_seed, "block_perm")
    perm = block_permutation(perm_key, num_blocks)
    table = np.full((B, spec.max_blocks), -1, dtype=np.int32)
    boff = np.concatenate([[0], np.cumsum(nblk)])
    for b in range(B):
        table[b, :nblk[b]] = perm[boff[b]:boff[b + 1]]
    store_dt = np.float32 if spec.dtype == "f32" else np.uint16
    kv = np.empty((num_blocks, BLOCK_SIZE, D), dtype=store_dt)
    if poison:
        kv[...] = _poison(spec.dtype)
    else:
        kv[...] = 0
    row_off = np.concatenate([[0], np.cumsum(np.maximum(lens, 0))])
    vs = spec.value_scale

    # Row chunks of at most CH rows (a whole number of blocks) per task.
    CH = 4096
    tasks = []
    for b in range(B):
        for r0 in range(0, int(max(lens[b], 0)), CH):
            tasks.append((b, r0, min(CH, int(lens[b]) - r0)))

    def work(t):
        b, r0, n = t
        st = store(_rows(spec, int(row_off[b]) + r0, n), spec.dtype)
        nb = (n + BLOCK_SIZE - 1) // BLOCK_SIZE
        k0 = r0 // BLOCK_SIZE
        for k in range(nb):
            pid = table[b, k0 + k]
            lo = k * BLOCK_SIZE
            hi = min(lo + BLOCK_SIZE, n)
            kv[pid, :hi - lo] = st[lo:hi]

    with ThreadPoolExecutor(max_workers=threads or _threads()) as ex:
        list(ex.map(work, tasks))

    H, T = spec.n_head, spec.t_q
    if spec.q_given:
        q_abs = _draw(spec, "q_abs", (B, T, H, D), vs)
        return Case(spec, lens.astype(np.int32), table, kv, None, None, None, None, q_abs)
    q_nope = _draw(spec, "q_nope", (B * T, H, spec.d_nope), vs)
    q_pe = _draw(spec, "q_pe", (B * T, H, R), vs)
    w_uk = _draw(spec, "w_uk", (H, spec.d_nope, Lk), spec.wscale())
    w_uv = _draw(spec, "w_uv", (H, spec.d_v, Lk), spec.wscale())
    return Case(spec, lens.astype(np.int32), table, kv, q_nope, q_pe, w_uk, w_uv, None)


def with_spec(spec: Spec, **kw) -> Spec:
    """A copy of a spec with some fields changed (smaller batches for tests)."""
    return replace(spec, **kw)


def sample_items(key_seed: int, batch: int, t_q: int, n_head: int, n: int,
                 must=()) -> np.ndarray:
    """n distinct (b, i, h) triples drawn uniformly, plus any listed ones."""
    total = batch * t_q * n_head
    n = min(n, total)
    order = np.argsort(draws(tensor_key(key_seed, "sample"), 0, total), kind="stable")[:n]
    items = set(int(x) for x in order)
    for (b, i, h) in must:
        items.add((b * t_q + i) * n_head + h)
    flat = np.array(sorted(items), dtype=np.int64)
    return np.stack([flat // (t_q * n_head), (flat // n_head) % t_q, flat % n_head], axis=1).astype(np.int32)


# --------------------------------------------------------------------------
# Cache-append prolog inputs
# --------------------------------------------------------------------------
# GLM-5.2 rope_theta, the base of the pages' rope permutation test.
ROPE_BASE = 8.0e6


@dataclass
class Append:
    """New tokens of one step, before RmsNorm and rope.  Storage arrays are
    float32 or bfloat16 bits (uint16), row-major."""
    c_kv: np.ndarray        # [n_tok][kv_rank], before RmsNorm
    k_pe: np.ndarray        # [n_tok][d_rope], before rope
    q_pe: np.ndarray        # [n_tok][H][d_rope], before rope
    gamma: np.ndarray       # [kv_rank]
    positions: np.ndarray   # int32 [n_tok]
    slots: np.ndarray       # int64 [n_tok] flat cache rows, -1 = padding token
    eps: float = RMS_EPS
    base: float = ROPE_BASE


def append_values(spec: Spec, n_tok: int, tag: str = "append") -> tuple:
    """(c_kv, k_pe, q_pe, gamma) of n_tok new tokens.  c_kv rows are
    N(0, 1) times a per-token log-normal magnitude exp(0.5 N(0, 1)), so row
    norms differ; gamma is 1 + 0.1 N(0, 1)."""
    Lk, R, H = spec.kv_rank, spec.d_rope, spec.n_head
    mag = np.exp(0.5 * normals(tensor_key(spec.seed, tag + ".mag"), 0, n_tok))
    c = normals(tensor_key(spec.seed, tag + ".c_kv"), 0, n_tok * Lk).reshape(n_tok, Lk) * mag[:, None]
    k = normals(tensor_key(spec.seed, tag + ".k_pe"), 0, n_tok * R).reshape(n_tok, R)
    q = normals(tensor_key(spec.seed, tag + ".q_pe"), 0, n_tok * H * R).reshape(n_tok, H, R)
    g = 1.0 + 0.1 * normals(tensor_key(spec.seed, tag + ".gamma"), 0, Lk)
    vs = spec.value_scale
    return (store(c * vs, spec.dtype), store(k * vs, spec.dtype), store(q * vs, spec.dtype),
            store(g, spec.dtype))


def step_append(spec: Spec, seq_lens, block_table, n_pad: int = 0, tag: str = "append") -> Append:
    """The new tokens of one decode step, request-major (b, i).

    seq_lens counts each request's rows including its t_q new ones, so query i
    of request b is logical row p = L - t_q + i, stored at flat cache row
    block_table[b][p // 16] * 16 + p % 16, with rope position p.  Requests
    shorter than t_q get padding slots (-1).  n_pad padding tokens (slot -1,
    position 0) follow, as when a batch is padded to a fixed size."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    B, T = lens.shape[0], spec.t_q
    n_tok = B * T + n_pad
    pos = np.zeros(n_tok, np.int32)
    slots = np.full(n_tok, -1, np.int64)
    for b in range(B):
        L = int(lens[b])
        if L < T:
            continue
        for i in range(T):
            p = L - T + i
            pos[b * T + i] = p
            slots[b * T + i] = int(block_table[b, p // BLOCK_SIZE]) * BLOCK_SIZE + p % BLOCK_SIZE
    c, k, q, g = append_values(spec, n_tok, tag)
    return Append(c, k, q, g, pos, slots)


def random_slots(key: int, num_slots: int, n_tok: int, n_skip: int = 0, n_out: int = 0) -> np.ndarray:
    """n_tok slot entries: distinct valid rows of [0, num_slots), with n_skip
    of them replaced by -1 and n_out by out-of-range rows (>= num_slots), at
    random places."""
    assert n_tok - n_skip - n_out <= num_slots
    valid = np.argsort(draws(key, 0, num_slots), kind="stable")[:n_tok].astype(np.int64)
    where = np.argsort(draws(key, num_slots, n_tok), kind="stable")
    valid[where[:n_skip]] = -1
    valid[where[n_skip:n_skip + n_out]] = num_slots + np.arange(n_out, dtype=np.int64) * 7
    return valid


def random_positions(key: int, n_tok: int, max_pos: int) -> np.ndarray:
    """int32 positions uniform in [0, max_pos]."""
    return np.floor(uniforms(key, 0, n_tok) * (max_pos + 1)).astype(np.int32)


# --------------------------------------------------------------------------
# Context-parallel shares
# --------------------------------------------------------------------------
def dcp_local(case: Case, world: int, rank: int, interleave: int = 1, seed: int = 7,
              spare_blocks: int = 2) -> tuple:
    """The paged cache rank `rank` of `world` holds when the rows of every
    request are dealt in runs of `interleave`: row j goes to rank
    (j // interleave) % world.  The rank keeps its rows in order as a request
    of its own in a fresh block pool (shuffled ids, NaN-poisoned spare blocks
    and tails).  Returns (kv_local, block_table_local, local_lens).  Data
    movement only: the stored values are copied unchanged."""
    s = case.spec
    lens = np.maximum(case.seq_lens.astype(np.int64), 0)
    rows_of = []
    for b in range(s.batch):
        j = np.arange(int(lens[b]))
        rows_of.append(j[(j // interleave) % world == rank])
    n_loc = np.array([len(r) for r in rows_of], dtype=np.int64)
    nblk = (n_loc + BLOCK_SIZE - 1) // BLOCK_SIZE
    max_blocks = int(max(1, nblk.max(initial=0)))
    num_blocks = int(nblk.sum()) + spare_blocks
    perm = block_permutation(tensor_key(seed + 131 * rank + 7919 * world, "dcp_perm"), num_blocks)
    table = np.full((s.batch, max_blocks), -1, dtype=np.int32)
    kv = np.empty((num_blocks, BLOCK_SIZE, s.D), dtype=case.kv.dtype)
    kv[...] = _poison(s.dtype)
    used = 0
    for b in range(s.batch):
        table[b, :nblk[b]] = perm[used:used + nblk[b]]
        used += int(nblk[b])
        for lj, gj in enumerate(rows_of[b]):
            gid = case.block_table[b, gj // BLOCK_SIZE]
            kv[table[b, lj // BLOCK_SIZE], lj % BLOCK_SIZE] = case.kv[gid, gj % BLOCK_SIZE]
    return kv, table, n_loc.astype(np.int32)


# --------------------------------------------------------------------------
# Fused prolog inputs
# --------------------------------------------------------------------------
PROLOG_HIDDEN, PROLOG_Q_RANK = 6144, 1536  # the pages fix neither; see the design notes


@dataclass
class PrologInputs:
    x: np.ndarray          # [n_tok][hidden]
    w_dq: np.ndarray       # [q_rank][hidden]
    w_uq: np.ndarray       # [H d_nope][q_rank]
    w_qr: np.ndarray       # [H d_rope][q_rank]
    w_dkv: np.ndarray      # [kv_rank][hidden]
    w_kr: np.ndarray       # [d_rope][hidden]
    gamma_q: np.ndarray    # [q_rank]
    gamma_kv: np.ndarray   # [kv_rank]


def prolog_inputs(spec: Spec, n_tok: int, hidden: int = PROLOG_HIDDEN, q_rank: int = PROLOG_Q_RANK,
                  tag: str = "prolog") -> PrologInputs:
    """Hidden states x ~ N(0, 1) (the output of the layer's input norm) and
    projection weights ~ N(0, 1) / sqrt(fan-in), stored [out][in] in the
    spec's dtype; norm gains 1 + 0.1 N(0, 1).  W_UK comes from the decode case
    of the same spec."""
    H, dn, dr, R = spec.n_head, spec.d_nope, spec.d_rope, spec.kv_rank

    def draw(name, shape, scale):
        n = int(np.prod(shape))
        return store_parallel(normals_parallel(tensor_key(spec.seed, f"{tag}_{name}"), n) * scale,
                              spec.dtype).reshape(shape)

    return PrologInputs(
        x=draw("x", (n_tok, hidden), 1.0),
        w_dq=draw("w_dq", (q_rank, hidden), 1.0 / math.sqrt(hidden)),
        w_uq=draw("w_uq", (H * dn, q_rank), 1.0 / math.sqrt(q_rank)),
        w_qr=draw("w_qr", (H * dr, q_rank), 1.0 / math.sqrt(q_rank)),
        w_dkv=draw("w_dkv", (R, hidden), 1.0 / math.sqrt(hidden)),
        w_kr=draw("w_kr", (dr, hidden), 1.0 / math.sqrt(hidden)),
        gamma_q=store(1.0 + 0.1 * normals(tensor_key(spec.seed, f"{tag}_gq"), 0, q_rank), spec.dtype),
        gamma_kv=store(1.0 + 0.1 * normals(tensor_key(spec.seed, f"{tag}_gkv"), 0, R), spec.dtype),
    )
