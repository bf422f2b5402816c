"""Parity of one rank's share of context-parallel decode
(mla_decode_attention_dcp) and of the LSE combine (mla_lse_combine), through
the C ABI, with the oracle.

Every rank's share is run on this one GPU from the paged cache that rank holds
(mla_inputs.dcp_local: rows dealt in runs of `interleave`, row j on rank
(j // interleave) % world) and compared with oracle.decode_share; the GPU
combine of all shares is compared with the oracle's full decode.  bf16
tolerances as the decode tests (tests/gpu_util.py); the combine on float32
inputs to 1e-5 relative.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import mla_latent_cache_amd as mla
import oracle
from gpu_util import DEV, assert_close, assert_lse_close, dims_tuple, oracle_dims, paged, to_dev, to_host

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on a GPU machine only
    pytest.skip("no GPU", allow_module_level=True)


def spec(base, **kw):
    return mi.with_spec(mi.SPECS[base], **kw)


def q_abs_for(case):
    """Absorbed queries on the device (GPU absorb, or the given ones) and the
    oracle's own [B][t_q][H][D] float64 copy."""
    s = case.spec
    dims = dims_tuple(s)
    sdt = torch.float32 if s.dtype == "f32" else torch.bfloat16
    if s.q_given:
        return to_dev(case.q_abs), case.q_abs
    q = torch.empty(s.batch, s.t_q, s.n_head, s.D, dtype=sdt, device=DEV)
    mla.mla_absorb_q(dims, to_dev(case.q_nope), to_dev(case.q_pe) if s.d_rope else None, to_dev(case.w_uk), q)
    q_o = oracle.absorb(oracle_dims(s), case.q_nope, case.q_pe, case.w_uk).reshape(s.batch, s.t_q, s.n_head, s.D)
    return q, q_o


def run_share(case, q_dev, world, rank, il, num_splits=0, out_dtype=torch.float32):
    s = case.spec
    dims = dims_tuple(s)
    kv, bt, _ = mi.dcp_local(case, world, rank, il)
    kv_d = to_dev(kv)
    bt_d = torch.from_numpy(bt).to(DEV)
    out = torch.empty(s.batch, s.t_q, s.n_head, s.kv_rank, dtype=out_dtype, device=DEV)
    lse = torch.empty(s.batch, s.t_q, s.n_head, dtype=torch.float32, device=DEV)
    ws = torch.empty(mla.mla_decode_workspace_size(dims, s.batch, s.t_q, bt.shape[1], 16, num_splits),
                     dtype=torch.uint8, device=DEV)
    mla.mla_decode_attention_dcp(dims, case.scale, q_dev, kv_d, bt_d, torch.from_numpy(case.seq_lens).to(DEV),
                                 world, rank, il, out, lse, ws, num_splits)
    torch.cuda.synchronize()
    return out, lse, mla.mla_decode_status(ws)


CASES = {
    "glm52_causal": dict(base="glm52_causal_tq4", batch=4, seq_len=0, fixed_lens=(300, 37, 0, 130), max_blocks=20,
                         spare_blocks=3),
    "tiny_f32": dict(base="tiny_f32", batch=3, fixed_lens=(5, 37, 0), max_blocks=3),
    "nope": dict(base="nope_long", batch=2, seq_len=0, fixed_lens=(517, 64), max_blocks=40, spare_blocks=2),
    "dsv3": dict(base="dsv3_ragged", batch=3, seq_len=0, fixed_lens=(700, 0, 33), zero_requests=(), max_blocks=48,
                 spare_blocks=2),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("world,il,splits", [(2, 1, 0), (4, 16, 0), (3, 5, 3), (8, 1, 2)])
def test_shares_and_combine(name, world, il, splits):
    kw = dict(CASES[name])
    case = mi.make_case(spec(kw.pop("base"), name=f"dcp_{name}", **kw))
    s = case.spec
    d = oracle_dims(s)
    q_dev, q_o = q_abs_for(case)
    outs, lses = [], []
    for r in range(world):
        out, lse, status = run_share(case, q_dev, world, r, il, splits)
        assert status == 0
        ref_o, ref_l, _ = oracle.decode_share(d, s.t_q, q_o, paged(case), case.scale, world, r, il)
        assert_close(to_host(out).reshape(-1, s.kv_rank), ref_o, s.dtype, f"rank {r} share")
        assert_lse_close(to_host(lse).reshape(-1), ref_l, s.dtype, f"rank {r} lse")
        outs.append(out)
        lses.append(lse)
    o_parts = torch.stack(outs).reshape(world, -1, s.kv_rank).contiguous()
    l_parts = torch.stack(lses).reshape(world, -1).contiguous()
    comb = torch.empty(o_parts.shape[1], s.kv_rank, dtype=torch.float32, device=DEV)
    comb_l = torch.empty(o_parts.shape[1], dtype=torch.float32, device=DEV)
    mla.mla_lse_combine(o_parts, l_parts, comb, comb_l)
    torch.cuda.synchronize()
    full_o, full_l, _ = oracle.decode(d, s.t_q, q_o, paged(case), case.scale)
    assert_close(to_host(comb), full_o, s.dtype, "combined shares vs full decode")
    assert_lse_close(to_host(comb_l), full_l, s.dtype, "combined lse vs full decode")


def test_world_one_is_plain_decode():
    case = mi.make_case(spec("glm52_causal_tq4", name="dcp_w1", batch=3, seq_len=0, fixed_lens=(90, 4, 250),
                             max_blocks=16, spare_blocks=2))  # = the blocks the longest needs, as in the rank's table
    s = case.spec
    dims = dims_tuple(s)
    q_dev, _ = q_abs_for(case)
    out1, lse1, _ = run_share(case, q_dev, 1, 0, 1)
    out2 = torch.empty_like(out1)
    lse2 = torch.empty_like(lse1)
    ws = torch.empty(mla.mla_decode_workspace_size(dims, s.batch, s.t_q, s.max_blocks, 16, 0), dtype=torch.uint8,
                     device=DEV)
    mla.mla_decode_attention(dims, case.scale, q_dev, to_dev(case.kv), torch.from_numpy(case.block_table).to(DEV),
                             torch.from_numpy(case.seq_lens).to(DEV), out2, lse2, ws)
    torch.cuda.synchronize()
    # the rank's cache is a relabelled copy of the request: same rows, same order
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_invalid_request_on_every_rank():
    case = mi.make_case(spec("glm52_causal_tq4", name="dcp_bad", batch=2, seq_len=0, fixed_lens=(64, 40),
                             max_blocks=5, spare_blocks=2))
    case.seq_lens[1] = 3  # 0 < L < t_q, judged on the global length
    s = case.spec
    q_dev, _ = q_abs_for(case)
    for r in range(3):
        out, lse, status = run_share(case, q_dev, 3, r, 1)
        assert status == mla.MLA_DATA_LEN_BELOW_TQ
        o = to_host(out)
        assert np.isnan(o[1]).all() and np.isfinite(o[0]).all() and np.isnan(to_host(lse)[1]).all()


def test_combine_kernel_against_oracle():
    rng = np.random.default_rng(9)
    P, n, W = 6, 37, 512
    o = rng.standard_normal((P, n, W)).astype(np.float32)
    l = (rng.standard_normal((P, n)) * 3).astype(np.float32)
    l[:, 3] = -np.inf                 # all parts empty
    l[2, 5] = -np.inf; o[2, 5] = np.nan  # an empty part's vector is not read
    l[4, 7] = np.nan                  # a NaN part poisons its row
    out = torch.empty(n, W, dtype=torch.float32, device=DEV)
    lse = torch.empty(n, dtype=torch.float32, device=DEV)
    mla.mla_lse_combine(to_dev(o), to_dev(l), out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.lse_combine(o, l)
    g, gl = to_host(out), to_host(lse)
    assert (g[3] == 0).all() and np.isneginf(gl[3])
    assert np.isnan(g[7]).all() and np.isnan(gl[7])
    ok = np.isfinite(ref_l)
    np.testing.assert_allclose(g[ok], ref_o[ok], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(gl[ok], ref_l[ok], rtol=1e-6, atol=1e-5)
    out_b = torch.empty(n, W, dtype=torch.bfloat16, device=DEV)
    mla.mla_lse_combine(to_dev(o), to_dev(l), out_b)
    torch.cuda.synchronize()
    assert_close(to_host(out_b)[ok], ref_o[ok], "bf16", "bf16 combine output")


def test_full_size_rank_share_sampled():
    # Rank 0 of 8 (interleave 1) at the GLM-5.2 decode size: 32 x 512 of the 4096 rows.
    case = mi.make_case(mi.SPECS["glm52_decode"])
    s = case.spec
    q_dev, q_o = q_abs_for(case)
    out, lse, status = run_share(case, q_dev, 8, 0, 1)
    assert status == 0
    sel = mi.sample_items(21, s.batch, s.t_q, s.n_head, 48, must=[(0, 0, 0), (31, 0, 63)])
    ref_o, ref_l, _ = oracle.decode_share(oracle_dims(s), s.t_q, q_o, paged(case), case.scale, 8, 0, 1, sel=sel)
    idx = (sel[:, 0] * s.t_q + sel[:, 1]) * s.n_head + sel[:, 2]
    assert_close(to_host(out).reshape(-1, s.kv_rank)[idx], ref_o, "bf16", "full-size rank share")
    assert_lse_close(to_host(lse).reshape(-1)[idx], ref_l, "bf16", "full-size rank lse")
