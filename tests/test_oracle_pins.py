"""Pins of the CPU oracle against what the pages and mathematics fix.

Each check compares the oracle with something outside it: golden values the
pages print (tests/golden/), a library routine the oracle never calls (torch's
scaled_dot_product_attention, numpy einsum, scipy logsumexp, numpy complex
arithmetic), the pages' own naive == absorbed identity, closed forms and
special cases.  The list is built so a plausible slip in the oracle -- a
dropped rope term, a wrong scale, a transposed W_UK, an off-by-one causal
horizon, the wrong V slice, a paging index error, a broken online rescale --
fails at least one test.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import mla_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def dims_of(spec):
    return oracle.Dims(spec.n_head, spec.d_nope, spec.d_rope, spec.d_v, spec.kv_rank)


def paged(case):
    return oracle.Paged(case.kv, case.block_table, case.seq_lens)


def small_spec(dims, t_q, lens, seed, dtype="f32", **kw):
    H, dn, dr, dv, r = dims
    mb = max(1, max((l + 15) // 16 for l in lens))
    return mi.Spec(f"pin_{seed}", H, dn, dr, dv, r, dtype, batch=len(lens), t_q=t_q,
                   max_blocks=mb + kw.pop("extra_blocks", 1), seed=seed, fixed_lens=tuple(lens),
                   spare_blocks=kw.pop("spare", 3), **kw)


def sdpa_reference(q_abs_bih, rows, kv_rank, t_q, scale):
    """torch SDPA (float64, CPU) of one request: q [t_q][H][D], rows [L][D].

    Causal rule of the mla.rs MlaInputs doc: query i sees rows 0 ..= L - t_q + i.
    Keys are the full rows, values their leading kv_rank columns.
    """
    t, H, D = q_abs_bih.shape
    L = rows.shape[0]
    q = torch.from_numpy(np.ascontiguousarray(q_abs_bih.transpose(1, 0, 2)))[None]  # [1,H,t,D]
    k = torch.from_numpy(rows)[None, None].expand(1, H, L, D).contiguous()
    v = torch.from_numpy(np.ascontiguousarray(rows[:, :kv_rank]))[None, None].expand(1, H, L, kv_rank).contiguous()
    mask = torch.zeros(t, L, dtype=torch.bool)
    for i in range(t):
        mask[i, :L - t_q + i + 1] = True
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()  # [t][H][kv_rank]


# --------------------------------------------------------------------------
# Golden constants
# --------------------------------------------------------------------------
def test_presets_and_scale_golden():
    g = golden("mla_presets.json")
    for name in ("GLM52", "GLM5_NEXT"):
        d = g[name]
        assert d["d_nope"] + d["d_rope"] == g["qk_head_dim_both"]
        assert d["kv_rank"] + d["d_rope"] == g["latent_row_width"][name]
        assert abs(oracle.scale(d["d_nope"], d["d_rope"]) - g["scale_both"]) <= g["scale_tol"]
    # the absorbed width must never reach the softmax
    d = g["GLM52"]
    assert abs(oracle.scale(d["d_nope"], d["d_rope"]) - 1 / math.sqrt(576)) > 1e-3
    # tiny geometry: 1/sqrt(16 + 8)
    assert abs(oracle.scale(16, 8) - 1 / math.sqrt(24)) < 1e-15
    v = golden("vllm_cpu_backend.json")
    assert v["kv_lora_rank"] + v["rope"] == v["head_size"] == g["latent_row_width"]["GLM52"]
    assert mi.BLOCK_SIZE == v["block_size"]


# --------------------------------------------------------------------------
# Absorb / decompress against numpy's einsum (a library routine the oracle never calls)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_absorb_matches_einsum(dtype):
    spec = small_spec((5, 12, 8, 10, 24), 2, [17, 3], seed=3, dtype=dtype)
    c = mi.make_case(spec)
    q_abs = oracle.absorb(dims_of(spec), c.q_nope, c.q_pe, c.w_uk)
    qn, qp, wuk = (mi.widen(a).astype(np.float64) for a in (c.q_nope, c.q_pe, c.w_uk))
    ref = np.concatenate([np.einsum("nhp,hpl->nhl", qn, wuk), qp], axis=-1)
    assert q_abs.shape == (4, 5, 32)
    np.testing.assert_allclose(q_abs, ref, rtol=1e-13, atol=1e-13)


def test_absorb_nope_geometry_has_no_rope_columns():
    spec = small_spec((3, 16, 0, 24, 48), 1, [5], seed=4)
    c = mi.make_case(spec)
    q_abs = oracle.absorb(dims_of(spec), c.q_nope, c.q_pe, c.w_uk)
    assert q_abs.shape == (1, 3, 48)
    ref = np.einsum("nhp,hpl->nhl", c.q_nope.astype(np.float64), c.w_uk.astype(np.float64))
    np.testing.assert_allclose(q_abs, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decompress_matches_einsum(dtype):
    spec = small_spec((5, 12, 8, 10, 24), 1, [9], seed=5, dtype=dtype)
    c = mi.make_case(spec)
    o_lat = mi.normals(99, 0, 7 * 5 * 24).reshape(7, 5, 24)
    out = oracle.decompress(dims_of(spec), o_lat, c.w_uv)
    ref = np.einsum("hjl,nhl->nhj", mi.widen(c.w_uv).astype(np.float64), o_lat)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("t_q,lens", [(1, [9, 0, 33]), (3, [5, 40])])
def test_attend_absorbed_is_the_composition_of_pinned_stages(dtype, t_q, lens):
    """The fused absorbed form equals absorb -> latent decode -> decompress,
    each of which is pinned on its own (einsum, einsum, torch SDPA)."""
    spec = small_spec((4, 12, 8, 10, 24), t_q, lens, seed=21 + t_q, dtype=dtype)
    c = mi.make_case(spec)
    d = dims_of(spec)
    out_f, o_f, lse_f, bad_f = oracle.attend_absorbed(d, t_q, c.q_nope, c.q_pe, c.w_uk, c.w_uv, paged(c), c.scale)
    assert bad_f == 0
    q_abs = oracle.absorb(d, c.q_nope, c.q_pe, c.w_uk).reshape(len(lens), t_q, spec.n_head, spec.D)
    o, lse, bad = oracle.decode(d, t_q, q_abs, paged(c), c.scale)
    assert bad == 0
    n = len(lens) * t_q
    out = oracle.decompress(d, o.reshape(n, spec.n_head, spec.kv_rank), c.w_uv).reshape(-1, spec.d_v)
    np.testing.assert_allclose(o_f, o.reshape(o_f.shape), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out_f, out, rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.isneginf(lse_f), np.isneginf(lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse_f[fin], lse[fin], rtol=1e-12, atol=1e-13)
    assert np.abs(out).max() > 1e-3  # not a vacuous comparison


# --------------------------------------------------------------------------
# Decode attention against torch SDPA on logically ordered rows
# --------------------------------------------------------------------------
@pytest.mark.parametrize("method", ["twopass", "online"])
@pytest.mark.parametrize("t_q,lens", [(1, [5, 37]), (3, [3, 20, 33]), (4, [16, 4])])
def test_decode_matches_sdpa(method, t_q, lens):
    spec = small_spec((4, 16, 8, 16, 32), t_q, lens, seed=11 + t_q, q_given=True)
    c = mi.make_case(spec)
    o, lse, bad = oracle.decode(dims_of(spec), t_q, c.q_abs, paged(c), c.scale, method=method)
    assert bad == 0
    H, R = spec.n_head, spec.kv_rank
    o = o.reshape(len(lens), t_q, H, R)
    for b, L in enumerate(lens):
        rows = mi.logical_rows(spec, c.seq_lens, b)
        ref = sdpa_reference(c.q_abs[b].astype(np.float64), rows, R, t_q, c.scale)
        np.testing.assert_allclose(o[b], ref, rtol=1e-12, atol=1e-13)


def test_decode_bf16_full_row_scores_match_sdpa():
    """bf16 storage, GLM-5.2-like row (rank 64, rope 64 scaled down): full-row keys."""
    spec = small_spec((8, 24, 16, 8, 64), 1, [40, 16, 1], seed=21, dtype="bf16", q_given=True)
    c = mi.make_case(spec)
    o, lse, bad = oracle.decode(dims_of(spec), 1, c.q_abs, paged(c), c.scale)
    o = o.reshape(3, 1, 8, 64)
    q = mi.widen(c.q_abs).astype(np.float64)
    for b in range(3):
        rows = mi.logical_rows(spec, c.seq_lens, b)
        ref = sdpa_reference(q[b], rows, 64, 1, c.scale)
        np.testing.assert_allclose(o[b], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("method", ["twopass", "online"])
def test_lse_matches_scipy_logsumexp(method):
    t_q, lens = 2, [7, 40]
    spec = small_spec((3, 16, 8, 16, 32), t_q, lens, seed=31, q_given=True)
    c = mi.make_case(spec)
    o, lse, bad = oracle.decode(dims_of(spec), t_q, c.q_abs, paged(c), c.scale, method=method)
    lse = lse.reshape(2, t_q, 3)
    for b, L in enumerate(lens):
        rows = mi.logical_rows(spec, c.seq_lens, b)
        for i in range(t_q):
            s = (c.q_abs[b, i].astype(np.float64) @ rows.T) * c.scale  # [H][L]
            n = L - t_q + i + 1
            ref = logsumexp(s[:, :n], axis=1)
            np.testing.assert_allclose(lse[b, i], ref, rtol=1e-13, atol=1e-13)
            # probabilities built from the oracle's lse sum to one
            np.testing.assert_allclose(np.exp(s[:, :n] - lse[b, i][:, None]).sum(1), 1.0, rtol=1e-12)


# --------------------------------------------------------------------------
# The pages' identity: naive form == absorbed form
# --------------------------------------------------------------------------
def _equiv_case(dims, t_q, t_kv, seed, tol, batch_lens=None):
    lens = batch_lens or [t_kv]
    spec = small_spec(tuple(dims), t_q, lens, seed=seed)
    c = mi.make_case(spec)
    d = dims_of(spec)
    naive, lse_n, bad_n = oracle.attend_naive(d, t_q, c.q_nope, c.q_pe, c.w_uk, c.w_uv, paged(c), c.scale)
    absd, o_lat, lse_a, bad_a = oracle.attend_absorbed(d, t_q, c.q_nope, c.q_pe, c.w_uk, c.w_uv,
                                                       paged(c), c.scale)
    assert bad_n == 0 and bad_a == 0
    md = np.abs(naive - absd).max()
    sc = max(np.abs(naive).max(), 1.0)
    assert md <= tol * sc                       # the page's own gate
    assert md <= 1e-11 * sc                     # float64 makes the identity far tighter
    np.testing.assert_allclose(lse_n, lse_a, rtol=1e-12, atol=1e-12)
    assert np.isfinite(naive).all() and np.abs(naive).max() > 1e-6


def test_naive_equals_absorbed_decode_page_shapes():
    g = golden("page_equivalence_cases.json")["decode_t1"]
    for k, dims in enumerate(g["dims"]):
        for seed in g["seeds"]:
            _equiv_case(dims, g["t_q"], g["t_kv"], seed + k, g["tol"])


def test_naive_equals_absorbed_prefill_causal_page_shapes():
    for cse in golden("page_equivalence_cases.json")["prefill_causal"]:
        _equiv_case(cse["dims"], cse["t_q"], cse["t_kv"], cse["seed"], cse["tol"])


def test_naive_equals_absorbed_glm52_full_dims():
    cse = golden("page_equivalence_cases.json")["glm52_full"]
    _equiv_case(cse["dims"], cse["t_q"], cse["t_kv"], cse["seed"], cse["tol"])


def test_naive_equals_absorbed_nope():
    g = golden("page_equivalence_cases.json")
    small = g["nope_small"]
    for k, dims in enumerate(small["dims"]):
        for seed in small["seeds"]:
            for cs in small["cases"]:
                _equiv_case(dims, cs["t_q"], cs["t_kv"], seed + cs["seed_offset"] + k, small["tol"])
    for cse in g["nope_full"]:
        _equiv_case(cse["dims"], cse["t_q"], cse["t_kv"], cse["seed"], cse["tol"])


def test_naive_equals_absorbed_multi_request_paged():
    """Several requests of different lengths in one shuffled paged cache."""
    _equiv_case((4, 24, 8, 32, 64), 2, None, 77, 1e-5, batch_lens=[2, 19, 33, 16])


# --------------------------------------------------------------------------
# Online recurrence == two-pass definition; special cases
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_f32"])
def test_online_equals_twopass_tiny(name):
    spec = mi.SPECS[name]
    c = mi.make_case(spec)
    d = dims_of(spec)
    q_abs = oracle.absorb(d, c.q_nope, c.q_pe, c.w_uk).reshape(spec.batch, spec.t_q, spec.n_head, spec.D)
    o2, l2, _ = oracle.decode(d, spec.t_q, q_abs, paged(c), c.scale, method="twopass")
    o1, l1, _ = oracle.decode(d, spec.t_q, q_abs, paged(c), c.scale, method="online")
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


def test_online_equals_twopass_causal_bf16():
    spec = small_spec((8, 16, 16, 8, 64), 4, [4, 31, 64, 17], seed=41, dtype="bf16", q_given=True)
    c = mi.make_case(spec)
    d = dims_of(spec)
    o2, l2, _ = oracle.decode(d, 4, c.q_abs, paged(c), c.scale, method="twopass")
    o1, l1, _ = oracle.decode(d, 4, c.q_abs, paged(c), c.scale, method="online")
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("method", ["twopass", "online"])
def test_single_row_returns_that_row(method):
    spec = small_spec((3, 8, 8, 8, 32), 1, [1, 1], seed=51, q_given=True)
    c = mi.make_case(spec)
    o, lse, _ = oracle.decode(dims_of(spec), 1, c.q_abs, paged(c), c.scale, method=method)
    for b in range(2):
        row = mi.logical_rows(spec, c.seq_lens, b)[0]
        for h in range(3):
            k = b * 3 + h
            np.testing.assert_array_equal(o[k], row[:32])
            s0 = float(c.q_abs[b, 0, h].astype(np.float64) @ row) * c.scale
            assert abs(lse[k] - s0) <= 1e-14 * max(1.0, abs(s0))


@pytest.mark.parametrize("method", ["twopass", "online"])
def test_identical_rows(method):
    """All rows equal: output is that row, lse = s + ln n."""
    spec = small_spec((2, 8, 8, 8, 32), 1, [23], seed=52, q_given=True, spare=1)
    c = mi.make_case(spec, poison=False)
    first = c.kv[c.block_table[0, 0], 0].copy()
    for k in range(2):
        c.kv[c.block_table[0, k]] = first
    o, lse, _ = oracle.decode(dims_of(spec), 1, c.q_abs, paged(c), c.scale, method=method)
    for h in range(2):
        np.testing.assert_allclose(o[h], first[:32].astype(np.float64), rtol=1e-14, atol=1e-15)
        s = float(c.q_abs[0, 0, h].astype(np.float64) @ first.astype(np.float64)) * c.scale
        assert abs(lse[h] - (s + math.log(23))) <= 1e-13


@pytest.mark.parametrize("method", ["twopass", "online"])
def test_empty_request_gives_zeros_and_neg_inf(method):
    spec = small_spec((4, 8, 8, 8, 32), 1, [0, 9, 0], seed=53, q_given=True)
    c = mi.make_case(spec)
    o, lse, bad = oracle.decode(dims_of(spec), 1, c.q_abs, paged(c), c.scale, method=method)
    o = o.reshape(3, 4, 32)
    lse = lse.reshape(3, 4)
    assert bad == 0
    for b in (0, 2):
        assert np.all(o[b] == 0.0) and not np.signbit(o[b]).any()
        assert np.all(np.isneginf(lse[b]))
    assert np.isfinite(o[1]).all() and np.isfinite(lse[1]).all()
    # full forms too
    spec2 = small_spec((4, 8, 8, 8, 32), 1, [0, 9], seed=54)
    c2 = mi.make_case(spec2)
    out, _, lse2, _ = oracle.attend_absorbed(dims_of(spec2), 1, c2.q_nope, c2.q_pe, c2.w_uk, c2.w_uv,
                                             paged(c2), c2.scale)
    assert np.all(out[:4] == 0.0) and np.all(np.isneginf(lse2[:4]))
    outn, lsen, _ = oracle.attend_naive(dims_of(spec2), 1, c2.q_nope, c2.q_pe, c2.w_uk, c2.w_uv,
                                        paged(c2), c2.scale)
    assert np.all(outn[:4] == 0.0) and np.all(np.isneginf(lsen[:4]))


@pytest.mark.parametrize("method", ["twopass", "online"])
def test_value_is_leading_kv_rank_slice(method):
    """With q_pe = 0 the rope columns add exact zeros to every score and must
    never enter the output: overwriting them leaves o_lat bit-identical."""
    spec = small_spec((4, 8, 16, 8, 32), 2, [21, 40], seed=55, q_given=True)
    c = mi.make_case(spec)
    c.q_abs[..., 32:] = 0.0
    o1, l1, _ = oracle.decode(dims_of(spec), 2, c.q_abs, paged(c), c.scale, method=method)
    kv2 = c.kv.copy()
    kv2[:, :, 32:] = 1e6
    c2 = oracle.Paged(kv2, c.block_table, c.seq_lens)
    o2, l2, _ = oracle.decode(dims_of(spec), 2, c.q_abs, c2, c.scale, method=method)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    assert o1.shape[1] == 32


def test_paging_relabel_is_bit_identical_and_poison_is_inert():
    spec = small_spec((4, 16, 8, 16, 32), 2, [3, 40, 17], seed=56, q_given=True, spare=5)
    c1 = mi.make_case(spec)
    c2 = mi.make_case(spec, relabel_seed=9999)
    assert not np.array_equal(c1.block_table, c2.block_table)
    for method in ("twopass", "online"):
        o1, l1, _ = oracle.decode(dims_of(spec), 2, c1.q_abs, paged(c1), c1.scale, method=method)
        o2, l2, _ = oracle.decode(dims_of(spec), 2, c2.q_abs, paged(c2), c2.scale, method=method)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)
        assert np.isfinite(o1).all()    # NaN spare blocks and tail rows never reached


def test_causal_query_equals_shorter_decode():
    """Query i of a t_q-token request equals a single-token decode whose
    request holds the first L - t_q + i + 1 rows."""
    t_q, L = 4, 37
    spec = small_spec((3, 8, 8, 8, 32), t_q, [L], seed=57, q_given=True)
    c = mi.make_case(spec)
    o, lse, _ = oracle.decode(dims_of(spec), t_q, c.q_abs, paged(c), c.scale)
    o = o.reshape(t_q, 3, 32)
    lse = lse.reshape(t_q, 3)
    for i in range(t_q):
        q1 = np.ascontiguousarray(c.q_abs[:, i:i + 1])
        c1 = oracle.Paged(c.kv, c.block_table, np.array([L - t_q + i + 1], np.int32))
        oi, li, _ = oracle.decode(dims_of(spec), 1, q1, c1, c.scale)
        np.testing.assert_array_equal(oi, o[i])
        np.testing.assert_array_equal(li, lse[i])


def test_invalid_requests_are_flagged_nan():
    spec = small_spec((2, 8, 8, 8, 32), 2, [5, 9, 20, 3, 8], seed=58, q_given=True)
    c = mi.make_case(spec)
    lens = c.seq_lens.copy()
    lens[0] = -1                                  # negative length
    lens[1] = spec.max_blocks * 16 + 1            # beyond the block-table row
    lens[3] = 1                                   # shorter than t_q
    bt = c.block_table.copy()
    bt[4, 0] = c.num_blocks                       # block id out of range
    cc = oracle.Paged(c.kv, bt, lens)
    o, lse, bad = oracle.decode(dims_of(spec), 2, c.q_abs, cc, c.scale)
    o = o.reshape(5, 2, 2, 32)
    assert bad == 4 * 2 * 2
    for b in (0, 1, 3, 4):
        assert np.isnan(o[b]).all()
    assert np.isfinite(o[2]).all()
    o2, _, bad2 = oracle.decode(dims_of(spec), 2, c.q_abs, cc, c.scale, method="online")
    assert bad2 == bad


def test_selection_matches_full():
    spec = small_spec((4, 16, 8, 16, 32), 2, [3, 40, 17], seed=59, q_given=True)
    c = mi.make_case(spec)
    o, lse, _ = oracle.decode(dims_of(spec), 2, c.q_abs, paged(c), c.scale)
    sel = np.array([[2, 1, 3], [0, 0, 0], [1, 1, 2]], np.int32)
    os_, ls, _ = oracle.decode(dims_of(spec), 2, c.q_abs, paged(c), c.scale, sel=sel)
    for k, (b, i, h) in enumerate(sel):
        idx = (b * 2 + i) * 4 + h
        np.testing.assert_array_equal(os_[k], o[idx])
        assert ls[k] == lse[idx]


# --------------------------------------------------------------------------
# RoPE pairings and the load-time permutation
# --------------------------------------------------------------------------
def test_norm_to_neox_perm_golden():
    g = golden("rope_permutation.json")
    np.testing.assert_array_equal(oracle.norm_to_neox_perm(8), g["perm_n8"])
    p = oracle.norm_to_neox_perm(64)
    assert sorted(p.tolist()) == list(range(64))


def test_rope_permutation_identity_page_test():
    g = golden("rope_permutation.json")
    n, base = g["n_dims"], g["base"]
    perm = oracle.norm_to_neox_perm(n)
    for k, pos in enumerate(g["positions"]):
        x0 = mi.normals(1000 + k, 0, n)
        y0 = mi.normals(2000 + k, 0, n)
        xa = oracle.rope_interleaved(x0, pos, base)
        xa_p = np.empty(n); xa_p[perm] = xa
        xb = np.empty(n); xb[perm] = x0
        xb = oracle.rope_neox(xb, pos, base)
        assert np.abs(xa_p - xb).max() <= g["tol_vec"]
        assert np.abs(xa_p - xb).max() <= 1e-12
        ya = oracle.rope_interleaved(y0, pos, base)
        yb = np.empty(n); yb[perm] = y0
        yb = oracle.rope_neox(yb, pos, base)
        dn, dx = float(xa @ ya), float(xb @ yb)
        assert abs(dn - dx) <= g["tol_dot"] * max(abs(dn), 1.0)


def test_rope_interleaved_is_complex_rotation():
    """Closed form: pairs as complex numbers times exp(i * pos * base^(-2j/n))."""
    n, base = 16, 10000.0
    x = mi.normals(7, 0, n)
    for pos in (0.0, 3.0, 123.5):
        th = pos * base ** (-2.0 * np.arange(n // 2) / n)
        z = (x[0::2] + 1j * x[1::2]) * np.exp(1j * th)
        ref = np.empty(n); ref[0::2] = z.real; ref[1::2] = z.imag
        np.testing.assert_allclose(oracle.rope_interleaved(x, pos, base), ref, rtol=1e-13, atol=1e-13)
        zn = (x[:n // 2] + 1j * x[n // 2:]) * np.exp(1j * th)
        refn = np.concatenate([zn.real, zn.imag])
        np.testing.assert_allclose(oracle.rope_neox(x, pos, base), refn, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(oracle.rope_interleaved(x, 0.0, base), x)
