"""Pins of the oracle's context-parallel pieces (decode_share, lse_combine)
against the mathematics, independent of the oracle's own code paths.

decode_share(world, rank, interleave) is one rank's share of decode context
parallelism: the vLLM CPU MLA backend page (CPUMLAImpl construction) carries
the settings dcp_world_size and cp_kv_cache_interleave_size; row j of a
request lives on rank (j // interleave) % world.  lse_combine is the split
merge.  The identity that pins both: combining the shares of all ranks gives
the full decode, for any world size and interleave, causal queries included.
"""
import numpy as np
import pytest
import scipy.special

import mla_inputs as mi
import oracle


def dims_of(s):
    return oracle.Dims(s.n_head, s.d_nope, s.d_rope, s.d_v, s.kv_rank)


def q_abs_of(case):
    s = case.spec
    return oracle.absorb(dims_of(s), case.q_nope, case.q_pe, case.w_uk).reshape(s.batch, s.t_q, s.n_head, s.D)


def paged(case):
    return oracle.Paged(case.kv, case.block_table, case.seq_lens)


CASES = {
    "tiny": mi.with_spec(mi.SPECS["tiny_f32"], name="dcp_tiny", batch=3, fixed_lens=(5, 37, 0), max_blocks=3),
    "causal": mi.with_spec(mi.SPECS["glm52_causal_tq4"], name="dcp_causal", n_head=4, batch=4, seq_len=0,
                           fixed_lens=(70, 4, 0, 33), max_blocks=5, spare_blocks=3),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("world,interleave", [(2, 1), (3, 5), (4, 16), (8, 1), (5, 7)])
def test_shares_combine_to_full_decode(name, world, interleave):
    case = mi.make_case(CASES[name])
    s = case.spec
    d, q, pg = dims_of(s), q_abs_of(case), paged(case)
    full_o, full_l, bad = oracle.decode(d, s.t_q, q, pg, case.scale)
    assert bad == 0
    parts = [oracle.decode_share(d, s.t_q, q, pg, case.scale, world, r, interleave) for r in range(world)]
    o, lse = oracle.lse_combine([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, full_o, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(full_l))
    fin = np.isfinite(full_l)
    np.testing.assert_allclose(lse[fin], full_l[fin], rtol=0, atol=1e-12)


def test_world_one_is_decode():
    case = mi.make_case(CASES["causal"])
    s = case.spec
    d, q, pg = dims_of(s), q_abs_of(case), paged(case)
    o1, l1, _ = oracle.decode(d, s.t_q, q, pg, case.scale)
    o2, l2, _ = oracle.decode_share(d, s.t_q, q, pg, case.scale, 1, 0, 3)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-14)


@pytest.mark.parametrize("world,rank,interleave", [(2, 1, 1), (3, 2, 5), (4, 0, 16)])
def test_share_equals_decode_of_the_ranks_rows(world, rank, interleave):
    # Brute force for one query per request: gather the rank's rows by hand
    # into a contiguous cache of their own and run the plain decode on it.
    spec = mi.with_spec(CASES["tiny"], t_q=1)
    case = mi.make_case(spec)
    s = case.spec
    d, q, pg = dims_of(s), q_abs_of(case), paged(case)
    got_o, got_l, _ = oracle.decode_share(d, 1, q, pg, case.scale, world, rank, interleave)
    for b in range(s.batch):
        L = int(case.seq_lens[b])
        rows = [j for j in range(L) if (j // interleave) % world == rank]
        if not rows:
            assert (got_o.reshape(s.batch, s.n_head, -1)[b] == 0).all()
            assert np.isneginf(got_l.reshape(s.batch, s.n_head)[b]).all()
            continue
        nb = (len(rows) + 15) // 16
        kv = np.zeros((nb, 16, s.D), case.kv.dtype)
        for lj, gj in enumerate(rows):
            kv[lj // 16, lj % 16] = case.kv[case.block_table[b, gj // 16], gj % 16]
        loc = oracle.Paged(kv, np.arange(nb, dtype=np.int32)[None, :], np.array([len(rows)], np.int32))
        ref_o, ref_l, _ = oracle.decode(d, 1, q[b:b + 1], loc, case.scale)
        np.testing.assert_allclose(got_o.reshape(s.batch, s.n_head, -1)[b], ref_o, rtol=0, atol=1e-14)
        np.testing.assert_allclose(got_l.reshape(s.batch, s.n_head)[b], ref_l, rtol=0, atol=1e-14)


def test_rank_without_rows_gives_zeros_and_minus_inf():
    case = mi.make_case(CASES["tiny"])  # request 0 has 5 rows: with interleave 16 rank 1 holds none
    s = case.spec
    o, l, _ = oracle.decode_share(dims_of(s), s.t_q, q_abs_of(case), paged(case), case.scale, 2, 1, 16)
    o = o.reshape(s.batch, s.n_head, -1)
    l = l.reshape(s.batch, s.n_head)
    assert (o[0] == 0).all() and np.isneginf(l[0]).all()


def test_invalid_request_is_nan_on_every_rank():
    case = mi.make_case(CASES["causal"])
    case.seq_lens[1] = 2  # 0 < L < t_q
    s = case.spec
    for r in range(3):
        o, l, bad = oracle.decode_share(dims_of(s), s.t_q, q_abs_of(case), paged(case), case.scale, 3, r, 1)
        o = o.reshape(s.batch, s.t_q, s.n_head, -1)
        assert bad == s.t_q * s.n_head and np.isnan(o[1]).all()


def test_combine_closed_forms():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((1, 4, 8))
    l = rng.standard_normal((1, 4))
    # P identical parts: same vectors, lse + ln P
    oc, lc = oracle.lse_combine(np.repeat(o, 3, 0), np.repeat(l, 3, 0))
    np.testing.assert_allclose(oc, o[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lc, l[0] + np.log(3), rtol=0, atol=1e-15)
    # a part with -inf LSE carries no weight, whatever its vector holds
    junk = np.full_like(o, np.nan)
    oc, lc = oracle.lse_combine(np.concatenate([o, junk]), np.concatenate([l, np.full_like(l, -np.inf)]))
    np.testing.assert_allclose(oc, o[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lc, l[0], rtol=0, atol=1e-15)
    # all parts empty: zeros and -inf; any NaN LSE: NaN
    oc, lc = oracle.lse_combine(junk, np.full_like(l, -np.inf))
    assert (oc == 0).all() and np.isneginf(lc).all()
    l2 = l.copy(); l2[0, 1] = np.nan
    oc, lc = oracle.lse_combine(o, l2)
    assert np.isnan(oc[1]).all() and np.isnan(lc[1]) and np.isfinite(lc[0])


def test_combine_weights_and_lse_against_logsumexp():
    rng = np.random.default_rng(4)
    P, n, R = 5, 6, 3
    o = rng.standard_normal((P, n, R))
    l = rng.standard_normal((P, n)) * 4
    oc, lc = oracle.lse_combine(o, l)
    np.testing.assert_allclose(lc, scipy.special.logsumexp(l, axis=0), rtol=0, atol=1e-13)
    w = scipy.special.softmax(l, axis=0)  # weights of the parts per row
    np.testing.assert_allclose(oc, np.einsum("pn,pnr->nr", w, o), rtol=0, atol=1e-13)


def test_dcp_local_holds_the_ranks_rows():
    # The input helper the GPU tests use: its local cache, read through its
    # table, is exactly the rank's rows in order.
    case = mi.make_case(CASES["causal"])
    kv, table, n_loc = mi.dcp_local(case, 3, 1, 5)
    for b in range(case.spec.batch):
        L = int(case.seq_lens[b])
        rows = [j for j in range(L) if (j // 5) % 3 == 1]
        assert n_loc[b] == len(rows)
        for lj, gj in enumerate(rows):
            got = kv[table[b, lj // 16], lj % 16]
            ref = case.kv[case.block_table[b, gj // 16], gj % 16]
            assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
