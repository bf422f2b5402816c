"""Parity of the cache-append prolog (mla_cache_append, through the C ABI) with
the oracle, on the GPU.

Every element of every written cache row and every rotated query element is
compared; rows the call must not touch are checked bit for bit.  Tolerances
follow from the arithmetic (float32 norm with a pairwise sum of squares, angles
formed in double and reduced before the float sine and cosine):
  float32 result:   |gpu - oracle| <= 4e-6 |oracle| + 2e-6 m
  bfloat16 result:  |gpu - oracle| <= 2^-8 |oracle| + 4e-6 m
where m = max(1, max |oracle| over the same row segment).  The bfloat16 term
is the half-unit rounding of the stored value.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import mla_latent_cache_amd as mla
import oracle
from gpu_util import (DeviceCase, assert_close, assert_lse_close, dims_tuple, oracle_dims, paged, run, to_dev,
                      to_host)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on a GPU machine only
    pytest.skip("no GPU", allow_module_level=True)

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
STYLES = {"neox": (oracle.NEOX, mla.MLA_ROPE_NEOX), "interleaved": (oracle.INTERLEAVED, mla.MLA_ROPE_INTERLEAVED)}


def check_segment(g, o, out_dt, what):
    """Row-segment comparison with the tolerance stated in the module doc."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU values"
    m = np.maximum(1.0, np.abs(o).max(axis=-1, keepdims=True))
    if out_dt == "f32":
        bound = 4e-6 * np.abs(o) + 2e-6 * m
    else:
        bound = 2.0 ** -8 * np.abs(o) + 4e-6 * m
    err = np.abs(g - o)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of tolerance, max err {err.max():.3e}"


def cache_tensor(num_blocks, D, dt, key):
    """A cache filled with seeded values, so untouched rows can be checked."""
    v = mi.store(mi.normals(key, 0, num_blocks * 16 * D).reshape(num_blocks, 16, D), dt)
    return v, to_dev(v)


def run_append(dims, ap_dev, cache_dev, style, err=None, q=True, gamma=True, eps=mi.RMS_EPS, base=mi.ROPE_BASE):
    c_kv, k_pe, q_pe, g, pos, slots = ap_dev
    mla.mla_cache_append(dims, c_kv, k_pe, g if gamma else None, eps, pos, base, style, q_pe if q else None,
                         slots, cache_dev, err)


def to_dev_append(c, k, q, g, pos, slots):
    return (to_dev(c), to_dev(k) if k is not None else None, to_dev(q) if q is not None else None, to_dev(g),
            torch.from_numpy(np.ascontiguousarray(pos, np.int32)).to("cuda"),
            torch.from_numpy(np.ascontiguousarray(slots, np.int64)).to("cuda"))


def oracle_append(cache_np, kv_rank, c, k, g, pos, style, slots, eps=mi.RMS_EPS, base=mi.ROPE_BASE):
    rows = mi.widen(cache_np).astype(np.float64).reshape(-1, cache_np.shape[-1]).copy()
    bad = oracle.cache_append(rows, kv_rank, c, k, g, eps, pos, base, style, slots)
    return rows, bad


def compare_cache(cache_dev, before_np, ref_rows, slots, kv_rank, out_dt):
    num_slots = ref_rows.shape[0]
    got = cache_dev.detach().float().cpu().numpy().astype(np.float64).reshape(num_slots, -1)
    before = mi.widen(before_np).astype(np.float64).reshape(num_slots, -1)
    written = np.unique(slots[(slots >= 0) & (slots < num_slots)])
    untouched = np.setdiff1d(np.arange(num_slots), written)
    np.testing.assert_array_equal(got[untouched], before[untouched])
    if written.size:
        check_segment(got[written, :kv_rank], ref_rows[written, :kv_rank], out_dt, "cache latent part")
        if ref_rows.shape[1] > kv_rank:
            check_segment(got[written, kv_rank:], ref_rows[written, kv_rank:], out_dt, "cache rope part")


# --------------------------------------------------------------------------
# Every element, GLM-5.2 geometry, both pairings, all dtype combinations
# --------------------------------------------------------------------------
@pytest.mark.parametrize("style", ["neox", "interleaved"])
@pytest.mark.parametrize("in_dt,kv_dt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")])
def test_cache_append_every_element(style, in_dt, kv_dt):
    o_style, g_style = STYLES[style]
    spec = mi.with_spec(mi.SPECS["glm52_decode"], dtype=in_dt)
    H, R, P = spec.n_head, spec.kv_rank, spec.d_rope
    n_tok, num_blocks = 37, 6                      # 37 tokens: a ragged last workgroup
    c, k, q, g = mi.append_values(spec, n_tok, tag="every")
    pos = mi.random_positions(91, n_tok, 131071)
    slots = mi.random_slots(93, num_blocks * 16, n_tok, n_skip=5, n_out=2)
    before, cache = cache_tensor(num_blocks, R + P, kv_dt, 95)
    dev = to_dev_append(c, k, q, g, pos, slots)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    run_append(dims_tuple(spec), dev, cache, g_style, err)
    torch.cuda.synchronize()
    ref_rows, bad = oracle_append(before, R, c, k, g, pos, o_style, slots)
    assert bad == 2
    assert int(err.item()) == mla.MLA_DATA_BAD_SLOT
    compare_cache(cache, before, ref_rows, slots, R, kv_dt)
    q_ref = oracle.rope_rows(q, pos, mi.ROPE_BASE, o_style)
    check_segment(to_host(dev[2]), q_ref, in_dt, "q_pe")


def test_cache_append_generic_path_odd_geometry():
    """kv_rank 36 and d_rope 10 take the element-wise kernel."""
    spec = mi.Spec("odd", 3, 8, 10, 8, 36, "bf16", batch=1, t_q=1, max_blocks=4, seed=611)
    n_tok, num_blocks = 9, 2
    for o_style, g_style in STYLES.values():
        c, k, q, g = mi.append_values(spec, n_tok)
        pos = mi.random_positions(97, n_tok, 5000)
        slots = mi.random_slots(99, num_blocks * 16, n_tok, n_skip=2)
        before, cache = cache_tensor(num_blocks, 46, "bf16", 101)
        dev = to_dev_append(c, k, q, g, pos, slots)
        run_append(dims_tuple(spec), dev, cache, g_style)
        torch.cuda.synchronize()
        ref_rows, _ = oracle_append(before, 36, c, k, g, pos, o_style, slots)
        compare_cache(cache, before, ref_rows, slots, 36, "bf16")
        check_segment(to_host(dev[2]), oracle.rope_rows(q, pos, mi.ROPE_BASE, o_style), "bf16", "q_pe")


def test_cache_append_unaligned_inputs_take_the_generic_path():
    """Inputs that start 2 bytes past a 16-byte boundary: same results."""
    spec = mi.SPECS["glm52_decode"]
    R, P, H = spec.kv_rank, spec.d_rope, spec.n_head
    n_tok, num_blocks = 6, 2
    c, k, q, g = mi.append_values(spec, n_tok, tag="unaligned")
    pos = mi.random_positions(103, n_tok, 70000)
    slots = mi.random_slots(105, num_blocks * 16, n_tok)
    before, cache = cache_tensor(num_blocks, R + P, "bf16", 107)

    def shifted(a):
        t = to_dev(a)
        big = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        v = big[1:].view(t.shape)
        v.copy_(t)
        return v

    dev = (shifted(c), shifted(k), shifted(q), to_dev(g),
           torch.from_numpy(pos).to("cuda"), torch.from_numpy(slots).to("cuda"))
    assert dev[0].data_ptr() % 16 != 0
    run_append(dims_tuple(spec), dev, cache, mla.MLA_ROPE_NEOX)
    torch.cuda.synchronize()
    ref_rows, _ = oracle_append(before, R, c, k, g, pos, oracle.NEOX, slots)
    compare_cache(cache, before, ref_rows, slots, R, "bf16")
    check_segment(to_host(dev[2]), oracle.rope_rows(q, pos, mi.ROPE_BASE, oracle.NEOX), "bf16", "q_pe")


def test_cache_append_no_gamma_no_queries_and_eps():
    spec = mi.SPECS["glm52_decode"]
    R, P = spec.kv_rank, spec.d_rope
    n_tok, num_blocks = 8, 1
    c, k, q, g = mi.append_values(spec, n_tok, tag="nogamma")
    pos = mi.random_positions(109, n_tok, 100)
    slots = mi.random_slots(111, 16, n_tok)
    before, cache = cache_tensor(num_blocks, R + P, "bf16", 113)
    dev = to_dev_append(c, k, q, g, pos, slots)
    q_before = dev[2].clone()
    run_append(dims_tuple(spec), dev, cache, mla.MLA_ROPE_NEOX, q=False, gamma=False, eps=0.5)
    torch.cuda.synchronize()
    assert torch.equal(dev[2], q_before)
    ref_rows, _ = oracle_append(before, R, c, k, None, pos, oracle.NEOX, slots, eps=0.5)
    compare_cache(cache, before, ref_rows, slots, R, "bf16")


def test_cache_append_nope_geometry_and_all_padding():
    spec = mi.SPECS["nope_long"]
    R = spec.kv_rank
    n_tok, num_blocks = 11, 2
    c, _, _, g = mi.append_values(spec, n_tok, tag="nope")
    slots = mi.random_slots(115, num_blocks * 16, n_tok, n_skip=3)
    before, cache = cache_tensor(num_blocks, R, "bf16", 117)
    mla.mla_cache_append(dims_tuple(spec), to_dev(c), None, to_dev(g), mi.RMS_EPS, None, 0.0, mla.MLA_ROPE_NEOX,
                         None, torch.from_numpy(slots).to("cuda"), cache)
    torch.cuda.synchronize()
    ref_rows, _ = oracle_append(before, R, c, None, g, None, oracle.NEOX, slots)
    compare_cache(cache, before, ref_rows, slots, R, "bf16")
    # Every token padding: nothing changes.
    snap = cache.clone()
    mla.mla_cache_append(dims_tuple(spec), to_dev(c), None, to_dev(g), mi.RMS_EPS, None, 0.0, mla.MLA_ROPE_NEOX,
                         None, torch.full((n_tok,), -1, dtype=torch.int64, device="cuda"), cache)
    torch.cuda.synchronize()
    assert torch.equal(cache, snap)


def test_cache_append_interleaved_equals_neox_on_permuted_rows():
    """The load-time permutation identity on the GPU: interleaved rope of x
    equals NEOX rope of the permuted x, permuted back."""
    spec = mi.SPECS["glm52_decode"]
    R, P, H = spec.kv_rank, spec.d_rope, spec.n_head
    n_tok = 16
    c, k, q, g = mi.append_values(spec, n_tok, tag="perm")
    pos = mi.random_positions(119, n_tok, 131071)
    slots = np.arange(n_tok, dtype=np.int64)
    perm = oracle.norm_to_neox_perm(P)
    k_p = np.empty_like(k); k_p[:, perm] = k
    q_p = np.empty_like(q); q_p[..., perm] = q
    outs = []
    for kk, qq, st in ((k, q, mla.MLA_ROPE_INTERLEAVED), (k_p, q_p, mla.MLA_ROPE_NEOX)):
        _, cache = cache_tensor(1, R + P, "f32", 121)
        dev = to_dev_append(c, kk, qq, g, pos, slots)
        run_append(dims_tuple(spec), dev, cache, st)
        torch.cuda.synchronize()
        outs.append((to_host(cache).reshape(16, R + P), to_host(dev[2])))
    (ci, qi), (cn, qn) = outs
    np.testing.assert_array_equal(ci[:, :R], cn[:, :R])
    np.testing.assert_allclose(ci[:, R:], cn[:, R + perm], rtol=0, atol=1e-6 * max(1, np.abs(ci).max()))
    np.testing.assert_allclose(qi, qn[..., perm], rtol=2.0 ** -7, atol=1e-6)  # one bf16 unit


# --------------------------------------------------------------------------
# The prolog feeding the decode path: append, then absorb + decode + decompress
# --------------------------------------------------------------------------
@pytest.mark.parametrize("base,kw", [
    ("glm52_decode", dict(batch=6, max_blocks=24, seq_len=0, fixed_lens=(300, 17, 1, 0, 64, 333))),
    ("glm52_causal_tq4", dict(batch=3, max_blocks=16, seq_len=0, fixed_lens=(100, 4, 250))),
])
def test_append_then_decode_step(base, kw):
    spec = mi.with_spec(mi.SPECS[base], **kw)
    case = mi.make_case(spec, poison=False)
    ap = mi.step_append(spec, case.seq_lens, case.block_table, n_pad=3)
    n_tok = spec.batch * spec.t_q
    dc = DeviceCase(case)
    # The step's new tokens: their q_pe rows are the case's own (pre-rope).
    q_pe_pre = case.q_pe
    dev = to_dev_append(ap.c_kv, ap.k_pe, np.concatenate([q_pe_pre, np.zeros((3,) + q_pe_pre.shape[1:],
                                                                                q_pe_pre.dtype)]),
                        ap.gamma, ap.positions, ap.slots)
    run_append(dims_tuple(spec), dev, dc.kv, mla.MLA_ROPE_NEOX)
    dc.q_pe = dev[2][:n_tok].contiguous()
    res = run(dc)
    assert res["status"] == 0

    # Oracle: the same append on its own copy of the cache, rope of the
    # queries, then the absorbed decode, all from the stored inputs.
    rows, _ = oracle_append(case.kv, spec.kv_rank, ap.c_kv, ap.k_pe, ap.gamma, ap.positions, oracle.NEOX,
                            ap.slots)
    kv_new = mi.store(rows.reshape(case.kv.shape), spec.dtype)
    q_pe_new = mi.store(oracle.rope_rows(q_pe_pre, ap.positions[:n_tok], mi.ROPE_BASE, oracle.NEOX), spec.dtype)
    cache_o = oracle.Paged(kv_new, case.block_table, case.seq_lens)
    d = oracle_dims(spec)
    out_ref, o_ref, lse_ref, bad = oracle.attend_absorbed(d, spec.t_q, case.q_nope, q_pe_new, case.w_uk,
                                                          case.w_uv, cache_o, case.scale)
    assert bad == 0
    assert_close(to_host(res["o_lat"]).reshape(-1, spec.kv_rank), o_ref, spec.dtype, "o_lat after append")
    assert_lse_close(to_host(res["lse"]).reshape(-1), lse_ref, spec.dtype, "lse after append")
    assert_close(to_host(res["out"]).reshape(-1, spec.d_v), out_ref, spec.dtype, "out after append")


# --------------------------------------------------------------------------
# Full sizes: the GLM-5.2 decode step's append, and a prefill-sized chunk
# --------------------------------------------------------------------------
def test_cache_append_glm52_decode_step_full_size():
    spec = mi.SPECS["glm52_decode"]
    case = mi.make_case(spec)
    ap = mi.step_append(spec, case.seq_lens, case.block_table)
    dc = DeviceCase(case)
    dev = to_dev_append(ap.c_kv, ap.k_pe, case.q_pe, ap.gamma, ap.positions, ap.slots)
    run_append(dims_tuple(spec), dev, dc.kv, mla.MLA_ROPE_NEOX)
    torch.cuda.synchronize()
    rows, _ = oracle_append(case.kv, spec.kv_rank, ap.c_kv, ap.k_pe, ap.gamma, ap.positions, oracle.NEOX,
                            ap.slots)
    compare_cache(dc.kv, case.kv, rows, ap.slots, spec.kv_rank, "bf16")
    check_segment(to_host(dev[2]), oracle.rope_rows(case.q_pe, ap.positions, mi.ROPE_BASE, oracle.NEOX), "bf16",
                  "q_pe")


def test_cache_append_prefill_chunk_4096_tokens():
    spec = mi.SPECS["glm52_decode"]
    R, P = spec.kv_rank, spec.d_rope
    n_tok, num_blocks = 4096, 320
    c, k, q, g = mi.append_values(spec, n_tok, tag="prefill")
    pos = np.arange(n_tok, dtype=np.int32) + 1000
    slots = mi.random_slots(123, num_blocks * 16, n_tok, n_skip=17)
    before, cache = cache_tensor(num_blocks, R + P, "bf16", 125)
    dev = to_dev_append(c, k, q, g, pos, slots)
    run_append(dims_tuple(spec), dev, cache, mla.MLA_ROPE_NEOX)
    torch.cuda.synchronize()
    ref_rows, _ = oracle_append(before, R, c, k, g, pos, oracle.NEOX, slots)
    compare_cache(cache, before, ref_rows, slots, R, "bf16")
    check_segment(to_host(dev[2]), oracle.rope_rows(q, pos, mi.ROPE_BASE, oracle.NEOX), "bf16", "q_pe")
