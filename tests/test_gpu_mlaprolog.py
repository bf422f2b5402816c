"""Parity of the fused prolog (mla_prolog, through the C ABI) with
oracle.prolog: the absorbed queries and the cache rows written, for small
projection widths and for the workload's (hidden 6144, q_rank 1536, the 32
tokens of a GLM-5.2 decode step).  bf16 tolerances as the decode tests; rows
the call must not touch are compared bit for bit."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import mla_latent_cache_amd as mla
import oracle
from gpu_util import DEV, assert_close, dims_tuple, oracle_dims, to_dev, to_host

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on a GPU machine only
    pytest.skip("no GPU", allow_module_level=True)


def run_case(spec, n_tok, hidden, q_rank, style=mla.MLA_ROPE_NEOX, n_pad=0, n_out=0, gammas=True, seed=3):
    case = mi.make_case(mi.with_spec(spec, batch=1, seq_len=0, fixed_lens=(16,), max_blocks=1, spare_blocks=0))
    p = mi.prolog_inputs(spec, n_tok, hidden, q_rank, tag=f"pt{seed}")
    num_blocks = (n_tok + 15) // 16 + 2
    slots = mi.random_slots(seed, num_blocks * 16, n_tok, n_skip=n_pad, n_out=n_out)
    pos = mi.random_positions(seed + 1, n_tok, 100000)
    D = spec.D
    cache0 = mi.store(np.random.default_rng(seed).standard_normal((num_blocks, 16, D)), "bf16")
    dims = dims_tuple(spec)
    dv = lambda a: to_dev(a) if a is not None else None
    kv = to_dev(cache0)
    q_abs = torch.empty(n_tok, spec.n_head, D, dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(mla.mla_prolog_workspace_size(dims, hidden, q_rank, n_tok), dtype=torch.uint8, device=DEV)
    gq = p.gamma_q if gammas else None
    gkv = p.gamma_kv if gammas else None
    mla.mla_prolog(dims, dv(p.x), dv(p.w_dq), dv(p.w_uq), dv(p.w_qr) if spec.d_rope else None, dv(case.w_uk),
                   dv(p.w_dkv), dv(p.w_kr) if spec.d_rope else None, dv(gq), dv(gkv), 1e-6, 1e-6,
                   torch.from_numpy(pos).to(DEV), mi.ROPE_BASE, style, torch.from_numpy(slots).to(DEV), kv, q_abs, ws,
                   err)
    torch.cuda.synchronize()
    rows = mi.widen(cache0).astype(np.float64).reshape(-1, D)
    ref_q, bad = oracle.prolog(oracle_dims(spec), p.x, p.w_dq, p.w_uq, p.w_qr, case.w_uk, p.w_dkv, p.w_kr, gq, gkv,
                               1e-6, 1e-6, pos, mi.ROPE_BASE, style, slots, rows)
    got_cache = to_host(kv).reshape(-1, D)
    written = np.zeros(rows.shape[0], bool)
    written[slots[(slots >= 0) & (slots < rows.shape[0])]] = True
    assert_close(to_host(q_abs).reshape(n_tok, -1), ref_q.reshape(n_tok, -1), "bf16", "absorbed queries")
    assert_close(got_cache[written], rows[written], "bf16", "written cache rows")
    assert np.array_equal(got_cache[~written], mi.widen(cache0).astype(np.float64).reshape(-1, D)[~written])
    assert (int(err.item()) & mla.MLA_DATA_BAD_SLOT != 0) == (bad > 0)
    return bad


GLM = mi.SPECS["glm52_decode"]


@pytest.mark.parametrize("n_tok", [1, 5, 40, 70])
def test_prolog_small_widths(n_tok):
    run_case(GLM, n_tok, hidden=256, q_rank=128, n_pad=min(2, n_tok - 1), seed=n_tok)


def test_prolog_interleaved_no_gains_and_bad_slots():
    bad = run_case(GLM, 24, hidden=512, q_rank=256, style=mla.MLA_ROPE_INTERLEAVED, n_pad=3, n_out=2, gammas=False)
    assert bad == 2


def test_prolog_nope_geometry():
    run_case(mi.SPECS["nope_long"], 17, hidden=384, q_rank=160, n_pad=1)


def test_prolog_decode_step_full_widths():
    run_case(GLM, 32, hidden=mi.PROLOG_HIDDEN, q_rank=mi.PROLOG_Q_RANK, seed=11)


def test_prolog_hip_graph_replay_matches_eager():
    # The fused prolog captured in one HIP graph and replayed three times, with
    # eager prolog calls on other inputs between the replays, writes the same
    # absorbed queries, cache rows and error word as the eager call, bit for bit.
    spec, n_tok, hidden, q_rank, seed = GLM, 40, 256, 128, 21
    case = mi.make_case(mi.with_spec(spec, batch=1, seq_len=0, fixed_lens=(16,), max_blocks=1, spare_blocks=0))
    p = mi.prolog_inputs(spec, n_tok, hidden, q_rank, tag="graph")
    num_blocks = (n_tok + 15) // 16 + 2
    slots = mi.random_slots(seed, num_blocks * 16, n_tok, n_skip=2, n_out=0)
    pos = torch.from_numpy(mi.random_positions(seed + 1, n_tok, 100000)).to(DEV)
    slots_d = torch.from_numpy(slots).to(DEV)
    cache0 = to_dev(mi.store(np.random.default_rng(seed).standard_normal((num_blocks, 16, spec.D)), "bf16"))
    dims = dims_tuple(spec)
    args = [to_dev(a) for a in (p.x, p.w_dq, p.w_uq, p.w_qr, case.w_uk, p.w_dkv, p.w_kr, p.gamma_q, p.gamma_kv)]
    ws = torch.empty(mla.mla_prolog_workspace_size(dims, hidden, q_rank, n_tok), dtype=torch.uint8, device=DEV)

    def call(kv, q_abs, err, stream=None):
        mla.mla_prolog(dims, *args, 1e-6, 1e-6, pos, mi.ROPE_BASE, mla.MLA_ROPE_NEOX, slots_d, kv, q_abs, ws, err,
                       stream)

    kv_e, q_e = cache0.clone(), torch.empty(n_tok, spec.n_head, spec.D, dtype=torch.bfloat16, device=DEV)
    err_e = torch.zeros(1, dtype=torch.int32, device=DEV)
    call(kv_e, q_e, err_e)
    torch.cuda.synchronize()
    kv_g, q_g = cache0.clone(), torch.empty_like(q_e)
    err_g = torch.zeros(1, dtype=torch.int32, device=DEV)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        call(kv_g, q_g, err_g, torch.cuda.current_stream())
    for rep in range(3):
        kv_g.copy_(cache0)
        q_g.zero_()
        err_g.zero_()
        g.replay()
        run_case(GLM, 5, hidden=256, q_rank=128, seed=9)  # eager work between replays (synchronises)
        torch.cuda.synchronize()
        assert torch.equal(q_g, q_e), rep
        assert torch.equal(kv_g, kv_e), rep
        assert torch.equal(err_g, err_e), rep
