"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Small cases compare every output element; the full-size workloads run in
the benchmark's launch configuration (automatic split count) and compare every
output (the DeepSeek-shaped one: every head of twelve requests, among them the
longest, the shortest and both empty ones).  Property tests cover split invariance, determinism, block relabelling,
the value slice, the causal mask, empty requests and device-side data errors.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import mla_latent_cache_amd as mla
import oracle
from gpu_util import (DEV, DeviceCase, assert_close, assert_lse_close, dims_tuple, flat_index, oracle_dims,
                      oracle_q_abs, paged, run, to_dev, to_host)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on a GPU machine only
    pytest.skip("no GPU", allow_module_level=True)


def spec_small(name, base, **kw):
    return mi.with_spec(mi.SPECS[base], name=name, **kw)


def full_compare(case, res, sel=None, naive_items=0):
    """Compare absorb, decode and decompress outputs of `res` with the oracle."""
    s = case.spec
    d = oracle_dims(s)
    if not s.q_given:
        qa = oracle_q_abs(case)
        assert_close(to_host(res["q_abs"]).reshape(qa.shape), qa, s.dtype, "q_abs")
    o_ref, lse_ref, bad = oracle.decode(d, s.t_q, oracle_q_abs(case), paged(case), case.scale, sel=sel)
    assert bad == 0
    idx = flat_index(s, sel) if sel is not None else slice(None)
    o_gpu = to_host(res["o_lat"]).reshape(-1, s.kv_rank)[idx]
    lse_gpu = to_host(res["lse"]).reshape(-1)[idx]
    assert_close(o_gpu, o_ref, s.dtype, "o_lat")
    assert_lse_close(lse_gpu, lse_ref, s.dtype, "lse")
    if not s.q_given:
        out_ref, o2, lse2, _ = oracle.attend_absorbed(d, s.t_q, case.q_nope, case.q_pe, case.w_uk, case.w_uv,
                                                      paged(case), case.scale, sel=sel)
        out_gpu = to_host(res["out"]).reshape(-1, s.d_v)[idx]
        assert_close(out_gpu, out_ref, s.dtype, "out")
        if naive_items:
            sel_n = sel[:naive_items] if sel is not None else mi.sample_items(7, s.batch, s.t_q, s.n_head,
                                                                              naive_items)
            out_n, _, _ = oracle.attend_naive(d, s.t_q, case.q_nope, case.q_pe, case.w_uk, case.w_uv,
                                              paged(case), case.scale, sel=sel_n)
            assert_close(to_host(res["out"]).reshape(-1, s.d_v)[flat_index(s, sel_n)], out_n, s.dtype,
                         "out vs naive form")


# --------------------------------------------------------------------------
# Small cases, every element
# --------------------------------------------------------------------------
@pytest.mark.parametrize("num_splits", [0, 1, 2, 3])
def test_tiny_f32_full_pipeline(num_splits):
    case = mi.make_case(mi.SPECS["tiny_f32"])
    res = run(DeviceCase(case), num_splits=num_splits)
    assert res["status"] == 0
    full_compare(case, res, naive_items=8)


SMALL = {
    "glm52_small": dict(base="glm52_decode", batch=5, fixed_lens=(1, 17, 100, 300, 64), max_blocks=20),
    "glm52_causal_small": dict(base="glm52_causal_tq4", batch=3, fixed_lens=(4, 35, 130), max_blocks=9),
    "nope_small": dict(base="nope_long", batch=3, fixed_lens=(33, 2, 257), max_blocks=17),
    "dsv3_small": dict(base="dsv3_ragged", batch=4, fixed_lens=(0, 50, 700, 16), max_blocks=44,
                       lengths="fixed", zero_requests=(0,)),
}


@pytest.mark.parametrize("num_splits", [1, 3, 0])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_bf16_every_element(name, num_splits):
    kw = dict(SMALL[name])
    spec = spec_small(name, kw.pop("base"), **kw)
    case = mi.make_case(spec)
    res = run(DeviceCase(case), num_splits=num_splits)
    assert res["status"] == 0
    full_compare(case, res, naive_items=0 if spec.q_given else 4)


def test_absorb_and_decompress_over_several_token_chunks():
    # 150 query rows (75 requests x 2 queries): the absorb and decompression
    # kernels give each group of 64 tokens its own workgroups, so this runs two
    # full groups and a ragged third one (22 rows: one full 16-row tile and 6
    # more); every element of q_abs, o_lat and out is compared.
    lens = tuple(2 + (7 * i) % 40 for i in range(75))
    spec = spec_small("glm52_many_tokens", "glm52_decode", batch=75, t_q=2, fixed_lens=lens, max_blocks=3)
    case = mi.make_case(spec)
    res = run(DeviceCase(case), num_splits=0)
    assert res["status"] == 0
    full_compare(case, res, naive_items=4)


def test_many_token_instances_give_the_same_bits():
    # A token's outputs are the same sequence of products whatever else the
    # call holds (the other tokens of its 64-token group, or other groups), so
    # the leading tokens of a wider call must match the narrower call bit for bit.
    torch.manual_seed(11)
    H, DN, R, DV, KR = 64, 192, 64, 256, 512
    dims = (H, DN, R, DV, KR)
    wuk = (torch.randn(H, DN, KR) * 0.05).bfloat16().to(DEV)
    wuv = (torch.randn(H, DV, KR) * 0.05).bfloat16().to(DEV)
    qn = torch.randn(150, H, DN).bfloat16().to(DEV)
    qp = torch.randn(150, H, R).bfloat16().to(DEV)
    ol = torch.randn(150, H, KR).bfloat16().to(DEV)
    for narrow_a, narrow_d in ((64, 32), (5, 17)):
        qa_w = torch.empty(150, H, KR + R, dtype=torch.bfloat16, device=DEV)
        qa_n = torch.empty(narrow_a, H, KR + R, dtype=torch.bfloat16, device=DEV)
        mla.mla_absorb_q(dims, qn, qp, wuk, qa_w)
        mla.mla_absorb_q(dims, qn[:narrow_a].contiguous(), qp[:narrow_a].contiguous(), wuk, qa_n)
        out_w = torch.empty(150, H, DV, dtype=torch.bfloat16, device=DEV)
        out_n = torch.empty(narrow_d, H, DV, dtype=torch.bfloat16, device=DEV)
        mla.mla_decompress_v(dims, ol, wuv, out_w)
        mla.mla_decompress_v(dims, ol[:narrow_d].contiguous(), wuv, out_n)
        torch.cuda.synchronize()
        assert torch.equal(qa_w[:narrow_a], qa_n)
        assert torch.equal(out_w[:narrow_d], out_n)


# (n_head, d_nope, d_rope, d_v, kv_rank): contraction lengths of 1, 3, 4, 6, 8
# and 16 k-steps of 32, rope widths copied 16 bytes (8, 64) or one element
# (4, 12) at a time or absent, d_v not a multiple of the 64-row slice.
GEMM_GEOMS = {
    "glm52": (64, 192, 64, 256, 512),
    "dsv3_heads16": (16, 128, 64, 128, 512),
    "ks3": (8, 96, 8, 64, 256),
    "ks16_nope": (4, 512, 0, 64, 512),
    "rope4_dv40": (4, 64, 4, 40, 128),
    "ks1_rope12": (3, 32, 12, 36, 64),
    # 256 or more (head, column slice) workgroups: absorb loops over the token
    # groups in one workgroup from 65 tokens on (rope copied element by
    # element; no rope with the longest contraction).
    "loop_rope12": (64, 32, 12, 36, 256),
    "loop_ks16_nope": (32, 512, 0, 64, 512),
}


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("n_tok", [1, 17, 64, 65, 150])
@pytest.mark.parametrize("geom", sorted(GEMM_GEOMS))
def test_absorb_and_decompress_every_element(geom, n_tok):
    """Every element of q_abs and out against the oracle's absorb and
    decompress, for bf16 and float32 outputs and float32 activations (which
    the kernels round to bf16 before the products, as the header states)."""
    H, DN, R, DV, KR = GEMM_GEOMS[geom]
    dims = (H, DN, R, DV, KR)
    d = oracle.Dims(H, DN, R, DV, KR)
    g = torch.Generator().manual_seed(1000 * n_tok + DN + R)
    qn = torch.randn(n_tok, H, DN, generator=g).bfloat16()
    qp = torch.randn(n_tok, H, R, generator=g).bfloat16()
    wuk = (torch.randn(H, DN, KR, generator=g) / DN ** 0.5).bfloat16()
    wuv = (torch.randn(H, DV, KR, generator=g) / KR ** 0.5).bfloat16()
    ol = torch.randn(n_tok, H, KR, generator=g)
    qa_ref = oracle.absorb(d, _bits(qn), _bits(qp), _bits(wuk))
    for odt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        qa = torch.empty(n_tok, H, KR + R, dtype=odt, device=DEV)
        mla.mla_absorb_q(dims, qn.to(DEV), qp.to(DEV) if R else None, wuk.to(DEV), qa)
        torch.cuda.synchronize()
        assert_close(to_host(qa), qa_ref, kind, f"q_abs ({odt})")
    ol_b = ol.bfloat16()
    out_ref = oracle.decompress(d, _bits(ol_b), _bits(wuv))
    for src in (ol_b, ol):
        for odt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
            out = torch.empty(n_tok, H, DV, dtype=odt, device=DEV)
            mla.mla_decompress_v(dims, src.to(DEV), wuv.to(DEV), out)
            torch.cuda.synchronize()
            assert_close(to_host(out), out_ref, kind, f"out ({src.dtype} in, {odt} out)")


def test_boundary_lengths_and_empty_requests():
    lens = (0, 1, 15, 16, 17, 31, 32, 33, 0, 63, 64, 65)
    spec = spec_small("glm52_edges", "glm52_decode", batch=len(lens), fixed_lens=lens, max_blocks=6)
    case = mi.make_case(spec)
    for num_splits in (1, 2, 4):
        res = run(DeviceCase(case), num_splits=num_splits, out_dtype=torch.float32)
        assert res["status"] == 0
        o = to_host(res["o_lat"])
        lse = to_host(res["lse"])
        out = to_host(res["out"]).reshape(len(lens), 1, spec.n_head, spec.d_v)
        for b in (0, 8):  # empty requests: exact zeros and -inf
            assert np.all(o[b] == 0.0) and not np.signbit(o[b]).any()
            assert np.all(np.isneginf(lse[b]))
            assert np.all(out[b] == 0.0)
        full_compare(case, res)


@pytest.mark.parametrize("num_splits", [64, 128])
def test_many_splits_wide_merge(num_splits):
    # 64 or more splits per request take the wide merge (a workgroup per query
    # row); a batch of 8 also takes the request-per-XCD mapping, and the empty
    # request and the short ones leave most of their ranges empty.
    lens = (1500, 0, 333, 17, 900, 64, 1, 2000)
    spec = spec_small("nope_many_splits", "nope_long", batch=len(lens), fixed_lens=lens, max_blocks=128)
    case = mi.make_case(spec)
    res = run(DeviceCase(case), num_splits=num_splits)
    assert res["status"] == 0
    assert np.all(to_host(res["o_lat"])[1] == 0.0) and np.all(np.isneginf(to_host(res["lse"])[1]))
    full_compare(case, res)


def test_hip_graph_replay_matches_eager():
    # The path captured in one HIP graph (absorb, split kernel, merge,
    # decompress) and replayed three times, with eager launches on other
    # inputs between the replays, reproduces the eager outputs bit for bit.
    lens = (1, 17, 100, 300, 64, 0, 33, 200)
    spec = spec_small("glm52_graph", "glm52_decode", batch=len(lens), fixed_lens=lens, max_blocks=20)
    case = mi.make_case(spec)
    dc = DeviceCase(case)
    ref = run(dc, num_splits=3)
    other = DeviceCase(mi.make_case(spec_small("glm52_graph_other", "glm52_decode", batch=2,
                                               fixed_lens=(50, 7), max_blocks=4)))
    dims = dims_tuple(spec)
    B, H, D, R = spec.batch, spec.n_head, spec.D, spec.kv_rank
    q_abs = torch.empty(B, 1, H, D, dtype=torch.bfloat16, device="cuda")
    out_lat = torch.empty(B, 1, H, R, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, 1, H, dtype=torch.float32, device="cuda")
    out = torch.empty(B, H, spec.d_v, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.mla_decode_workspace_size(dims, B, 1, dc.bt.shape[1], 16, 3), dtype=torch.uint8,
                     device="cuda")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        st = torch.cuda.current_stream()
        mla.mla_absorb_q(dims, dc.q_nope, dc.q_pe, dc.w_uk, q_abs, st)
        mla.mla_decode_attention(dims, case.scale, q_abs, dc.kv, dc.bt, dc.sl, out_lat, lse, ws, 3, st)
        mla.mla_decompress_v(dims, out_lat, dc.w_uv, out, st)
    for rep in range(3):
        for t in (q_abs, out_lat, out):
            t.zero_()
        lse.fill_(7.0)
        g.replay()
        run(other, num_splits=2)  # eager work between replays
        torch.cuda.synchronize()
        assert mla.mla_decode_status(ws) == 0
        assert torch.equal(q_abs, ref["q_abs"]), rep
        assert torch.equal(out_lat, ref["o_lat"]), rep
        assert torch.equal(lse, ref["lse"]), rep
        assert torch.equal(out, ref["out"]), rep


# --------------------------------------------------------------------------
# Full-size workloads, launch configuration of the benchmark, sampled outputs
# --------------------------------------------------------------------------
# Full-size workloads and the number of sampled items also checked against
# the naive (per-head decompression) form.
FULL = {"glm52_decode": 2, "dsv3_ragged": 0, "glm52_causal_tq4": 2, "nope_long": 0, "nope_wide": 2}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size(name):
    # Every (request, query, head) output of the GLM-5.2, causal and NoPE
    # workloads; for the DeepSeek-shaped one, every head of the longest, the
    # shortest non-empty, both empty and eight seeded other requests.
    spec = mi.SPECS[name]
    case = mi.make_case(spec)
    res = run(DeviceCase(case), num_splits=0)
    assert res["status"] == 0
    sel = None
    if name == "dsv3_ragged":
        lens = case.seq_lens.astype(np.int64)
        longest = int(np.argmax(lens))
        shortest = int(np.argmin(np.where(lens > 0, lens, np.iinfo(np.int64).max)))
        others = [int(b) for b in np.argsort(mi.draws(mi.tensor_key(spec.seed, "test_requests"), 0, spec.batch))
                  if b not in (0, 63, longest, shortest)][:8]
        reqs = sorted({0, 63, longest, shortest, *others})
        sel = np.array([(b, 0, h) for b in reqs for h in range(spec.n_head)], dtype=np.int32)
    naive = mi.sample_items(spec.seed, spec.batch, spec.t_q, spec.n_head, FULL[name]) if FULL[name] else None
    full_compare(case, res, sel=sel, naive_items=0)
    if naive is not None:
        d = oracle_dims(spec)
        out_n, _, _ = oracle.attend_naive(d, spec.t_q, case.q_nope, case.q_pe, case.w_uk, case.w_uv, paged(case),
                                          case.scale, sel=naive)
        assert_close(to_host(res["out"]).reshape(-1, spec.d_v)[flat_index(spec, naive)], out_n, spec.dtype,
                     "out vs naive form")
    if name == "dsv3_ragged":  # every head of the two empty requests
        o = to_host(res["o_lat"])
        lse = to_host(res["lse"])
        for b in (0, 63):
            assert np.all(o[b] == 0.0) and np.all(np.isneginf(lse[b]))
    assert np.isfinite(to_host(res["o_lat"])[case.seq_lens > 0]).all()


def test_one_long_request_and_many_short_every_element():
    # The length-balanced schedule: one 32768-row request among 63 short ones
    # (some empty) is cut across many workgroups while the short ones are
    # finished whole; every output element is compared.
    short = [int(x) for x in (mi.uniforms(mi.tensor_key(77, "short_lens"), 0, 63) * 301).astype(np.int64)]
    short[5] = short[40] = 0
    lens = tuple([32768] + short)
    spec = spec_small("dsv3_long_short", "dsv3_ragged", batch=64, fixed_lens=lens, max_blocks=2048,
                      lengths="fixed", zero_requests=())
    case = mi.make_case(spec)
    for k in (0, 2):
        res = run(DeviceCase(case), num_splits=k)
        assert res["status"] == 0
        full_compare(case, res)


@pytest.mark.parametrize("batch", [8, 16])
@pytest.mark.parametrize("num_splits", [2, 5, 16])
def test_batch_multiple_of_8_every_element(batch, num_splits):
    # With a batch that is a multiple of 8 the split kernel and the merge map
    # request b to XCD b % 8; every element is compared.
    lens = tuple(17 + (97 * b) % 700 for b in range(batch))
    spec = spec_small(f"glm52_b{batch}", "glm52_decode", batch=batch, fixed_lens=lens, max_blocks=48)
    case = mi.make_case(spec)
    res = run(DeviceCase(case), num_splits=num_splits)
    assert res["status"] == 0
    full_compare(case, res)


def test_flat_schedule_split_invariance_and_determinism():
    # 128 query rows per request (the length-balanced kernel): results for
    # different range counts (including many more ranges than tiles, which
    # leaves ranges empty) agree within rounding, and each is reproducible.
    spec = spec_small("dsv3_mid", "dsv3_ragged", batch=5, fixed_lens=(700, 0, 1000, 33, 257), max_blocks=64,
                      lengths="fixed", zero_requests=())
    case = mi.make_case(spec)
    dc = DeviceCase(case)
    outs = {}
    for k in (1, 2, 7, 0, 64):
        r1 = run(dc, num_splits=k, out_dtype=torch.float32)
        r2 = run(dc, num_splits=k, out_dtype=torch.float32)
        assert r1["status"] == 0
        assert torch.equal(r1["o_lat"], r2["o_lat"]) and torch.equal(r1["lse"], r2["lse"]), k
        outs[k] = (to_host(r1["o_lat"]), to_host(r1["lse"]))
    ref, lref = outs[1]
    fin = np.isfinite(lref)
    for k, (o, l) in outs.items():
        assert np.abs(o - ref).max() <= 2e-3 * np.abs(ref).max(), k
        assert np.array_equal(np.isneginf(l), np.isneginf(lref))
        assert np.abs(l[fin] - lref[fin]).max() <= 1e-4 * max(1.0, np.abs(lref[fin]).max()), k
    full_compare(case, run(dc, num_splits=64))


@pytest.mark.parametrize("heads,t_q", [(32, 1), (16, 2), (8, 4)])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_split_kernel_below_64_query_rows_every_element(heads, t_q, num_splits):
    # Fewer than 64 query rows per request (heads x queries) take the
    # per-request split kernel instead of the length-balanced one; GLM-5.2
    # head dimensions, causal multi-token queries, every element compared.
    lens = (700, 0, 1000, 33, 257)
    spec = spec_small(f"glm52_h{heads}_t{t_q}", "glm52_decode", n_head=heads, t_q=t_q, batch=len(lens),
                      fixed_lens=lens, max_blocks=64)
    case = mi.make_case(spec)
    res = run(DeviceCase(case), num_splits=num_splits)
    assert res["status"] == 0
    full_compare(case, res)


@pytest.mark.parametrize("base", ["dsv3_ragged", "glm52_decode"])
def test_score_growth_far_past_the_first_tile_every_element(base):
    # 128 (DeepSeek-shaped) or 64 (GLM-5.2) query rows per request.  The rope
    # columns of late rows of two requests are scaled by 200, so their scores exceed those of the request's first tile by far more than
    # the length-balanced kernel's fixed softmax reference allows (64 in log2 units):
    # the pieces holding the jump are streamed a second time with their true
    # maximum.  A third request grows by 18-41 (no second pass; probabilities
    # up to 2^41 before normalisation).  The value columns are untouched.
    # Every element is compared, for range counts that cut the requests at
    # different places.
    spec = spec_small(f"{base}_growth", base, batch=4, fixed_lens=(700, 1000, 33, 257), max_blocks=64,
                      lengths="fixed", zero_requests=())
    case = mi.make_case(spec)
    kv = mi.bf16_bits_to_f32(case.kv)
    for b, lo, f in ((1, 300, 200.0), (0, 100, 12.0), (3, 200, 200.0)):
        for j in range(lo, int(case.seq_lens[b])):
            kv[case.block_table[b, j // 16], j % 16, spec.kv_rank:] *= f
    case.kv[...] = mi.to_bf16_bits(kv)
    for k in (1, 3, 0):
        res = run(DeviceCase(case), num_splits=k)
        assert res["status"] == 0
        full_compare(case, res)


@pytest.mark.parametrize("base", ["dsv3_ragged", "glm52_decode"])
def test_second_pass_covers_rows_other_than_the_first_every_element(base):
    # Only some query rows see a jump: the rope columns of late rows of request
    # 1 are scaled by 200, and the rope part of the queries of heads 0, 32, 64
    # and 96 (the first row of each 32-row wave) is zero, so those rows' scores
    # do not grow while every other row's do.  Any row past the softmax
    # reference's limit must send the workgroup round a second time.
    spec = spec_small(f"{base}_quiet", base, batch=3, fixed_lens=(700, 1000, 257), max_blocks=64,
                      lengths="fixed", zero_requests=())
    case = mi.make_case(spec)
    kv = mi.bf16_bits_to_f32(case.kv)
    for j in range(300, int(case.seq_lens[1])):
        kv[case.block_table[1, j // 16], j % 16, spec.kv_rank:] *= 200.0
    case.kv[...] = mi.to_bf16_bits(kv)
    quiet = list(range(0, spec.n_head, 32))
    if spec.q_given:
        case.q_abs[:, :, quiet, spec.kv_rank:] = 0
    else:
        case.q_pe[:, quiet, :] = 0
    for k in (1, 3, 5, 0):
        res = run(DeviceCase(case), num_splits=k)
        assert res["status"] == 0
        full_compare(case, res)


# --------------------------------------------------------------------------
# Properties
# --------------------------------------------------------------------------
def mid_case(**kw):
    spec = spec_small("glm52_mid", "glm52_decode", batch=4, fixed_lens=(700, 1000, 33, 257), max_blocks=64, **kw)
    return mi.make_case(spec)


def test_split_invariance_and_determinism():
    case = mid_case()
    dc = DeviceCase(case)
    outs = {}
    for k in (1, 2, 7, 0, 64):
        r1 = run(dc, num_splits=k, out_dtype=torch.float32)
        r2 = run(dc, num_splits=k, out_dtype=torch.float32)
        a, b = to_host(r1["o_lat"]), to_host(r2["o_lat"])
        assert np.array_equal(a, b), f"num_splits={k}: two runs differ"
        assert np.array_equal(to_host(r1["lse"]), to_host(r2["lse"]))
        outs[k] = (a, to_host(r1["lse"]))
    ref, lref = outs[1]
    scale = np.abs(ref).max()
    for k, (o, l) in outs.items():
        # different ranges change where bf16 probabilities are rounded and the f32 sum order
        assert np.abs(o - ref).max() <= 2e-3 * scale, k
        assert np.abs(l - lref).max() <= 1e-4 * max(1.0, np.abs(lref).max()), k


def test_relabelled_blocks_bit_identical():
    case = mid_case()
    case2 = mi.make_case(case.spec, relabel_seed=4242)
    assert not np.array_equal(case.block_table, case2.block_table)
    for k in (1, 3):
        r1 = run(DeviceCase(case), num_splits=k)
        r2 = run(DeviceCase(case2), num_splits=k)
        for key in ("o_lat", "lse", "out"):
            assert torch.equal(r1[key], r2[key]), (k, key)


def test_value_is_leading_kv_rank_slice():
    spec = spec_small("dsv3_vslice", "dsv3_ragged", batch=3, fixed_lens=(40, 300, 17), max_blocks=19,
                      lengths="fixed", zero_requests=())
    case = mi.make_case(spec)
    case.q_abs[..., 512:] = 0  # rope part of the queries zero: k_pe adds exact zeros to every score
    r1 = run(DeviceCase(case), num_splits=2)
    kv2 = case.kv.copy()
    live = np.isfinite(mi.widen(kv2))
    big = mi.to_bf16_bits(np.full(kv2[..., 512:].shape, 3.0e4, np.float32))
    kv2[..., 512:] = np.where(live[..., 512:], big, kv2[..., 512:])
    case2 = mi.Case(case.spec, case.seq_lens, case.block_table, kv2, None, None, None, None, case.q_abs)
    r2 = run(DeviceCase(case2), num_splits=2)
    assert torch.equal(r1["o_lat"], r2["o_lat"])
    assert torch.equal(r1["lse"], r2["lse"])


def test_causal_mask_probe():
    spec = spec_small("causal_probe", "glm52_causal_tq4", batch=2, fixed_lens=(37, 200), max_blocks=13)
    case = mi.make_case(spec)
    r1 = run(DeviceCase(case), num_splits=1)
    kv2 = case.kv.copy()
    for b, L in enumerate(case.seq_lens):
        j = int(L) - 1  # the last row: visible only to the last query of request b
        kv2[case.block_table[b, j // 16], j % 16, :] = mi.to_bf16_bits(np.full(spec.D, 2.5, np.float32))
    case2 = mi.Case(case.spec, case.seq_lens, case.block_table, kv2, case.q_nope, case.q_pe, case.w_uk,
                    case.w_uv, None)
    r2 = run(DeviceCase(case2), num_splits=1)
    o1, o2 = r1["o_lat"], r2["o_lat"]
    assert torch.equal(o1[:, :3], o2[:, :3]), "queries 0..t_q-2 must not see the last row"
    assert not torch.equal(o1[:, 3], o2[:, 3])


def test_data_errors_flag_and_poison_only_their_request():
    spec = spec_small("errs", "glm52_causal_tq4", batch=6, fixed_lens=(40, 40, 40, 40, 40, 40), max_blocks=4)
    case = mi.make_case(spec)
    dc = DeviceCase(case)
    clean = run(dc, num_splits=2, out_dtype=torch.float32)
    assert clean["status"] == 0
    lens = case.seq_lens.copy()
    lens[0] = -3                       # negative length
    lens[1] = 4 * 16 + 1               # beyond the block-table row
    lens[2] = 2                        # fewer rows than queries
    bt = case.block_table.copy()
    bt[3, 1] = case.num_blocks + 5     # block id out of range
    bt[4, 2] = -7                      # negative block id inside the request
    res = run(dc, num_splits=2, out_dtype=torch.float32, seq_lens=torch.from_numpy(lens).cuda(),
              block_table=torch.from_numpy(bt).cuda())
    assert res["status"] == (mla.MLA_DATA_NEG_LEN | mla.MLA_DATA_LEN_OVER_TABLE | mla.MLA_DATA_LEN_BELOW_TQ
                             | mla.MLA_DATA_BAD_BLOCK)
    o = to_host(res["o_lat"])
    for b in range(5):
        assert np.isnan(o[b]).all(), b
        assert np.isnan(to_host(res["lse"])[b]).all(), b
    assert torch.equal(res["o_lat"][5], clean["o_lat"][5])
    again = run(dc, num_splits=2, out_dtype=torch.float32)
    assert again["status"] == 0 and torch.equal(again["o_lat"], clean["o_lat"])
