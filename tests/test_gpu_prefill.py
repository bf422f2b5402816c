"""Parity of the naive-form prefill path (mla_prefill_attention, through the C
ABI) with the oracle, on the GPU.

The oracle's naive form (per-head decompression of every visible row) is the
reference for a seeded sample of (request, query, head) items; the oracle's
absorbed form, which the pages prove equal and which is cheap enough, covers
every item.  Tolerance: the bf16 bar of the decode tests (|gpu - oracle| <=
2e-2 + 1e-2 |oracle| elementwise and <= 1e-2 max |oracle| overall).  The GPU
path rounds the decompressed K_nope and V rows to bf16 in its workspace; the
oracle keeps them in float64.
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


def run_prefill(case, out_dtype=torch.bfloat16):
    s = case.spec
    dims = dims_tuple(s)
    B, T, H = s.batch, s.t_q, s.n_head
    q_nope = to_dev(case.q_nope).view(B, T, H, s.d_nope)
    q_pe = to_dev(case.q_pe).view(B, T, H, s.d_rope) if s.d_rope else None
    out = torch.empty(B, T, H, s.d_v, dtype=out_dtype, device=DEV)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=DEV)
    ws = torch.empty(mla.mla_prefill_workspace_size(dims, B, s.max_blocks), dtype=torch.uint8, device=DEV)
    mla.mla_prefill_attention(dims, case.scale, q_nope, q_pe, to_dev(case.w_uk), to_dev(case.w_uv), to_dev(case.kv),
                              torch.from_numpy(case.block_table).to(DEV), torch.from_numpy(case.seq_lens).to(DEV),
                              out, lse, ws)
    torch.cuda.synchronize()
    return out, lse, mla.mla_decode_status(ws)


def compare(case, out, lse, naive_items=48, seed=5):
    s = case.spec
    d = oracle_dims(s)
    ref, _, ref_lse, bad = oracle.attend_absorbed(d, s.t_q, case.q_nope, case.q_pe, case.w_uk, case.w_uv,
                                                  paged(case), case.scale)
    valid = np.array([0 <= L <= s.max_blocks * 16 and not (0 < L < s.t_q) for L in case.seq_lens])
    rows = np.repeat(valid, s.t_q * s.n_head)
    got = to_host(out).reshape(-1, s.d_v)
    got_lse = to_host(lse).reshape(-1)
    assert np.isnan(got[~rows]).all() and np.isnan(got_lse[~rows]).all()
    assert_close(got[rows], ref[rows], "bf16", "prefill out vs absorbed oracle")
    assert_lse_close(got_lse[rows], ref_lse[rows], "bf16", "prefill lse vs absorbed oracle")
    vb = np.nonzero(valid)[0]
    if naive_items and vb.size:
        sel = mi.sample_items(seed, s.batch, s.t_q, s.n_head, naive_items)
        sel = sel[np.isin(sel[:, 0], vb)]
        out_n, lse_n, _ = oracle.attend_naive(d, s.t_q, case.q_nope, case.q_pe, case.w_uk, case.w_uv, paged(case),
                                              case.scale, sel=sel)
        idx = (sel[:, 0] * s.t_q + sel[:, 1]) * s.n_head + sel[:, 2]
        assert_close(got[idx], out_n, "bf16", "prefill out vs naive oracle")
        assert_lse_close(got_lse[idx], lse_n, "bf16", "prefill lse vs naive oracle")
    return bad


def spec(base, **kw):
    return mi.with_spec(mi.SPECS[base], **kw)


@pytest.mark.parametrize("lens,t_q", [((300, 37, 130), 8), ((160, 200), 160), ((33, 64, 1), 1), ((130, 130), 130)])
def test_prefill_glm52_chunked_and_full(lens, t_q):
    s = spec("glm52_causal_tq4", name="pf", batch=len(lens), t_q=t_q, seq_len=0, fixed_lens=lens,
             max_blocks=max((l + 15) // 16 for l in lens) + 1, spare_blocks=3)
    case = mi.make_case(s)
    out, lse, status = run_prefill(case)
    assert status == 0
    compare(case, out, lse)


def test_prefill_nope_geometry():
    s = spec("nope_long", name="pf_nope", batch=2, t_q=40, seq_len=0, fixed_lens=(100, 77), max_blocks=8,
             spare_blocks=2)
    case = mi.make_case(s)
    out, lse, status = run_prefill(case)
    assert status == 0
    compare(case, out, lse)


def test_prefill_two_heads():
    # 2 heads: the stacked [W_UK; W_UV] is 384 + 512 rows, seven 128-row weight
    # tiles, a single XCD group, so most of the decompression's workgroups have
    # no tile and leave at once.
    s = spec("glm52_causal_tq4", name="pf_h2", n_head=2, batch=2, t_q=33, seq_len=0, fixed_lens=(300, 77),
             max_blocks=20, spare_blocks=3)
    case = mi.make_case(s)
    out, lse, status = run_prefill(case)
    assert status == 0
    compare(case, out, lse)


def test_prefill_f32_output_and_edge_requests():
    # Request 1 is empty (zeros, -inf); request 2 is shorter than t_q (NaN and a status bit).
    s = spec("glm52_causal_tq4", name="pf_edge", batch=4, t_q=20, seq_len=0, fixed_lens=(45, 0, 7, 20),
             max_blocks=4, spare_blocks=2)
    case = mi.make_case(s)
    out, lse, status = run_prefill(case, out_dtype=torch.float32)
    assert status == mla.MLA_DATA_LEN_BELOW_TQ
    compare(case, out, lse)
    got = to_host(out)
    assert (got[1] == 0).all() and np.isneginf(to_host(lse)[1]).all()


def test_prefill_ragged_query_tiles():
    # t_q = 257: three 128-query tiles, the last with one query; rows not a
    # multiple of the 32-row tile.
    s = spec("glm52_causal_tq4", name="pf_ragged", batch=1, t_q=257, seq_len=0, fixed_lens=(301,), max_blocks=20,
             spare_blocks=3)
    case = mi.make_case(s)
    out, lse, status = run_prefill(case)
    assert status == 0
    compare(case, out, lse, naive_items=32)


def test_prefill_bad_block_is_flagged():
    s = spec("glm52_causal_tq4", name="pf_badblk", batch=2, t_q=4, seq_len=0, fixed_lens=(40, 40), max_blocks=3,
             spare_blocks=2)
    case = mi.make_case(s)
    case.block_table[1, 1] = case.num_blocks + 5  # outside the cache
    out, lse, status = run_prefill(case)
    assert status == mla.MLA_DATA_BAD_BLOCK
    got = to_host(out)
    assert np.isnan(got[1]).all() and np.isfinite(got[0]).all()


def test_prefill_full_size_sampled():
    # The benchmark's prefill workload: 2 requests x 4096 rows, 1024 new queries each.
    s = mi.SPECS["glm52_prefill"]
    case = mi.make_case(s)
    out, lse, status = run_prefill(case)
    assert status == 0
    d = oracle_dims(s)
    sel = mi.sample_items(11, s.batch, s.t_q, s.n_head, 24, must=[(0, 0, 0), (1, s.t_q - 1, s.n_head - 1)])
    ref, _, ref_lse, _ = oracle.attend_absorbed(d, s.t_q, case.q_nope, case.q_pe, case.w_uk, case.w_uv, paged(case),
                                                case.scale, sel=sel)
    idx = (sel[:, 0] * s.t_q + sel[:, 1]) * s.n_head + sel[:, 2]
    assert_close(to_host(out).reshape(-1, s.d_v)[idx], ref, "bf16", "full-size prefill out")
    assert_lse_close(to_host(lse).reshape(-1)[idx], ref_lse, "bf16", "full-size prefill lse")


def test_prefill_hip_graph_replay_matches_eager():
    # The call captured in one HIP graph and replayed three times, with eager
    # calls on other inputs between the replays, reproduces the eager outputs
    # bit for bit (the call's first kernel clears the status words each time).
    s = spec("glm52_causal_tq4", name="pf_graph", batch=2, t_q=40, seq_len=0, fixed_lens=(130, 77), max_blocks=10,
             spare_blocks=2)
    case = mi.make_case(s)
    ref_out, ref_lse, status = run_prefill(case)
    assert status == 0
    other = mi.make_case(spec("glm52_causal_tq4", name="pf_graph_other", batch=1, t_q=8, seq_len=0, fixed_lens=(50,),
                              max_blocks=4, spare_blocks=1))
    dims = dims_tuple(s)
    B, T, H = s.batch, s.t_q, s.n_head
    q_nope = to_dev(case.q_nope).view(B, T, H, s.d_nope)
    q_pe = to_dev(case.q_pe).view(B, T, H, s.d_rope)
    w_uk, w_uv, kv = to_dev(case.w_uk), to_dev(case.w_uv), to_dev(case.kv)
    bt, sl = torch.from_numpy(case.block_table).to(DEV), torch.from_numpy(case.seq_lens).to(DEV)
    out = torch.empty(B, T, H, s.d_v, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=DEV)
    ws = torch.empty(mla.mla_prefill_workspace_size(dims, B, s.max_blocks), dtype=torch.uint8, device=DEV)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        mla.mla_prefill_attention(dims, case.scale, q_nope, q_pe, w_uk, w_uv, kv, bt, sl, out, lse, ws,
                                  torch.cuda.current_stream())
    for rep in range(3):
        out.zero_()
        lse.fill_(7.0)
        g.replay()
        _, _, other_status = run_prefill(other)  # eager work between replays
        torch.cuda.synchronize()
        assert other_status == 0
        assert mla.mla_decode_status(ws) == 0
        assert torch.equal(out, ref_out), rep
        assert torch.equal(lse, ref_lse), rep
