"""The C-ABI library on the host: it loads, exports every declared entry point,
and rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import math
import os
import re

import pytest

import mla_latent_cache_amd as mla
from mla_latent_cache_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 8
    L = mla.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/mla.h but not exported"
    assert set(names) == set(B.EXPORTS)


GLM52 = (64, 192, 64, 256, 512)
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def dims(t=GLM52):
    return ctypes.byref(B.mla_dims(*t))


def decode(**kw):
    a = dict(dims=dims(), scale=0.0625, batch=2, t_q=1, q=FAKE, kv=FAKE, dt=B.MLA_BF16, num_blocks=10,
             block_size=16, bt=FAKE, max_blocks=4, sl=FAKE, out=FAKE, out_dt=B.MLA_BF16, lse=None,
             ws=FAKE, ws_bytes=1 << 30, splits=1, stream=None)
    a.update(kw)
    return mla.lib().mla_decode_attention(a["dims"], a["scale"], a["batch"], a["t_q"], a["q"], a["kv"], a["dt"],
                                          a["num_blocks"], a["block_size"], a["bt"], a["max_blocks"], a["sl"],
                                          a["out"], a["out_dt"], a["lse"], a["ws"], a["ws_bytes"], a["splits"],
                                          a["stream"])


def test_decode_host_validation():
    assert decode(dims=None) == B.MLA_ERR_NULL
    assert decode(dims=dims((0, 192, 64, 256, 512))) == B.MLA_ERR_DIMS
    assert decode(dims=dims((64, 192, -1, 256, 512))) == B.MLA_ERR_DIMS
    assert decode(dims=dims((64, 192, 64, 256, 0))) == B.MLA_ERR_DIMS
    assert decode(batch=-1) == B.MLA_ERR_SHAPE
    assert decode(t_q=0) == B.MLA_ERR_SHAPE
    assert decode(max_blocks=0) == B.MLA_ERR_SHAPE
    assert decode(num_blocks=0) == B.MLA_ERR_SHAPE
    assert decode(splits=-2) == B.MLA_ERR_SHAPE
    assert decode(block_size=8) == B.MLA_ERR_UNSUPPORTED
    assert decode(block_size=32) == B.MLA_ERR_UNSUPPORTED
    assert decode(dt=7) == B.MLA_ERR_ARG
    assert decode(out_dt=2) == B.MLA_ERR_ARG
    assert decode(scale=0.0) == B.MLA_ERR_ARG
    assert decode(scale=-1.0) == B.MLA_ERR_ARG
    assert decode(scale=math.nan) == B.MLA_ERR_ARG
    assert decode(scale=math.inf) == B.MLA_ERR_ARG
    assert decode(ws=None) == B.MLA_ERR_NULL
    assert decode(q=None) == B.MLA_ERR_NULL
    assert decode(kv=None) == B.MLA_ERR_NULL
    assert decode(bt=None) == B.MLA_ERR_NULL
    assert decode(sl=None) == B.MLA_ERR_NULL
    assert decode(out=None) == B.MLA_ERR_NULL
    assert decode(ws_bytes=16, splits=4) == B.MLA_ERR_WORKSPACE


def test_decode_refuses_misaligned_pointers():
    # 16-byte vectors for the queries, cache and outputs; 4-byte words for the
    # table, lengths and LSE; a 256-byte aligned workspace.
    odd16 = ctypes.c_void_p(0x1008)
    odd4 = ctypes.c_void_p(0x1002)
    assert decode(q=odd16) == B.MLA_ERR_ARG
    assert decode(kv=odd16) == B.MLA_ERR_ARG
    assert decode(out=odd16) == B.MLA_ERR_ARG
    assert decode(bt=odd4) == B.MLA_ERR_ARG
    assert decode(sl=odd4) == B.MLA_ERR_ARG
    assert decode(lse=odd4) == B.MLA_ERR_ARG
    assert decode(ws=ctypes.c_void_p(0x1080)) == B.MLA_ERR_ARG
    L = mla.lib()
    assert L.mla_absorb_q(dims(), 4, odd16, FAKE, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_ARG
    assert L.mla_absorb_q(dims(), 4, FAKE, odd16, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_ARG
    assert L.mla_absorb_q(dims(), 4, FAKE, FAKE, FAKE, 1, odd16, 1, None) == B.MLA_ERR_ARG
    assert L.mla_decompress_v(dims(), 4, odd16, 1, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_ARG
    assert L.mla_decompress_v(dims(), 4, FAKE, 1, FAKE, 1, odd16, 1, None) == B.MLA_ERR_ARG


def test_decode_refuses_plans_beyond_32bit_counts():
    # Workgroup and status-slot counts are 32-bit on the device: a plan whose
    # count would wrap is refused instead of launching a wrong grid.
    sz = ctypes.c_size_t()
    L = mla.lib()
    big = (65536, 1, 0, 1, 32)  # generic path (float32 geometry): one workgroup per query row
    assert L.mla_decode_workspace_size(dims(big), 1024, 1, 4096, 16, 1024, ctypes.byref(sz)) == B.MLA_ERR_SHAPE
    assert decode(dims=dims(big), batch=1024, max_blocks=4096, splits=1024, dt=B.MLA_F32) == B.MLA_ERR_SHAPE


def test_workspace_size_explicit_splits():
    sz = ctypes.c_size_t()
    L = mla.lib()
    assert L.mla_decode_workspace_size(dims(), 32, 1, 256, 16, 1, ctypes.byref(sz)) == B.MLA_OK
    one = sz.value
    assert one >= 256 and one % 256 == 0
    assert L.mla_decode_workspace_size(dims(), 32, 1, 256, 16, 8, ctypes.byref(sz)) == B.MLA_OK
    eight = sz.value
    # eight splits need per-split (o, lse) partials: 32 * 8 * 64 * (512 + 1) float32 at least
    assert eight >= 32 * 8 * 64 * 513 * 4 and eight > one
    assert L.mla_decode_workspace_size(dims(), 32, 1, 256, 8, 8, ctypes.byref(sz)) == B.MLA_ERR_UNSUPPORTED
    assert L.mla_decode_workspace_size(dims(), 32, 0, 256, 16, 8, ctypes.byref(sz)) == B.MLA_ERR_SHAPE
    assert L.mla_decode_workspace_size(dims(), 32, 1, 256, 16, 8, None) == B.MLA_ERR_NULL
    # bf16 MFMA geometry: the batch's tiles are cut into batch * num_splits ranges
    assert L.mla_decode_resolve_splits(dims(), 32, 1, 256, 8) == 256
    assert L.mla_decode_resolve_splits(dims(), 32, 1, 256, 7) == 224
    assert L.mla_decode_resolve_splits(dims(), 32, 0, 256, 8) == 0
    # other geometries: whole-block ranges of every request (37 blocks per range, 7 ranges)
    tiny = (4, 16, 8, 16, 32)
    assert L.mla_decode_resolve_splits(dims(tiny), 32, 1, 256, 7) == 32 * 7
    assert L.mla_decode_resolve_splits(dims(tiny), 32, 1, 256, 500) == 32 * 256


def test_absorb_and_decompress_host_validation():
    L = mla.lib()
    assert L.mla_absorb_q(None, 4, FAKE, FAKE, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_NULL
    assert L.mla_absorb_q(dims((64, 0, 64, 256, 512)), 4, FAKE, FAKE, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_DIMS
    assert L.mla_absorb_q(dims(), -1, FAKE, FAKE, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_SHAPE
    assert L.mla_absorb_q(dims(), 4, FAKE, FAKE, FAKE, 3, FAKE, 1, None) == B.MLA_ERR_ARG
    assert L.mla_absorb_q(dims(), 4, FAKE, None, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_NULL  # rope needed
    assert L.mla_absorb_q(dims(), 0, None, None, None, 1, None, 1, None) == B.MLA_OK          # empty: no-op
    assert L.mla_decompress_v(None, 4, FAKE, 1, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_NULL
    assert L.mla_decompress_v(dims((64, 192, 64, 0, 512)), 4, FAKE, 1, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_DIMS
    assert L.mla_decompress_v(dims(), -3, FAKE, 1, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_SHAPE
    assert L.mla_decompress_v(dims(), 4, FAKE, 1, FAKE, 9, FAKE, 1, None) == B.MLA_ERR_ARG
    assert L.mla_decompress_v(dims(), 4, None, 1, FAKE, 1, FAKE, 1, None) == B.MLA_ERR_NULL
    assert L.mla_decode_status(None, None, None) == B.MLA_ERR_NULL


def append(**kw):
    a = dict(dims=dims(), n_tok=4, c_kv=FAKE, k_pe=FAKE, gamma=None, in_dt=B.MLA_BF16, eps=1e-6, pos=FAKE,
             base=8e6, style=B.MLA_ROPE_NEOX, q_pe=FAKE, slots=FAKE, cache=FAKE, kv_dt=B.MLA_BF16,
             num_blocks=10, block_size=16, err=None, stream=None)
    a.update(kw)
    return mla.lib().mla_cache_append(a["dims"], a["n_tok"], a["c_kv"], a["k_pe"], a["gamma"], a["in_dt"],
                                      a["eps"], a["pos"], a["base"], a["style"], a["q_pe"], a["slots"],
                                      a["cache"], a["kv_dt"], a["num_blocks"], a["block_size"], a["err"],
                                      a["stream"])


def test_cache_append_host_validation():
    assert append(dims=None) == B.MLA_ERR_NULL
    assert append(dims=dims((64, 192, 64, 256, 0))) == B.MLA_ERR_DIMS
    assert append(dims=dims((64, 192, -2, 256, 512))) == B.MLA_ERR_DIMS
    assert append(dims=dims((64, 192, 63, 256, 512))) == B.MLA_ERR_DIMS   # odd rope width
    assert append(dims=dims((0, 192, 64, 256, 512))) == B.MLA_ERR_DIMS    # heads needed for q_pe
    assert append(n_tok=-1) == B.MLA_ERR_SHAPE
    assert append(num_blocks=0) == B.MLA_ERR_SHAPE
    assert append(block_size=32) == B.MLA_ERR_UNSUPPORTED
    assert append(dims=dims((64, 192, 258, 256, 512))) == B.MLA_ERR_UNSUPPORTED
    assert append(in_dt=5) == B.MLA_ERR_ARG
    assert append(kv_dt=-1) == B.MLA_ERR_ARG
    assert append(eps=-1e-6) == B.MLA_ERR_ARG
    assert append(eps=math.nan) == B.MLA_ERR_ARG
    assert append(eps=math.inf) == B.MLA_ERR_ARG
    assert append(base=0.0) == B.MLA_ERR_ARG
    assert append(base=math.inf) == B.MLA_ERR_ARG
    assert append(style=2) == B.MLA_ERR_ARG
    assert append(c_kv=None) == B.MLA_ERR_NULL
    assert append(slots=None) == B.MLA_ERR_NULL
    assert append(cache=None) == B.MLA_ERR_NULL
    assert append(k_pe=None) == B.MLA_ERR_NULL
    assert append(pos=None) == B.MLA_ERR_NULL
    assert append(n_tok=0, c_kv=None, k_pe=None, pos=None, q_pe=None, slots=None, cache=None) == B.MLA_OK
    # No rope part: k_pe, positions and rope base are not needed.
    nope = (64, 256, 0, 256, 512)
    assert append(dims=dims(nope), n_tok=0, k_pe=None, pos=None, base=0.0) == B.MLA_OK


def prefill(**kw):
    a = dict(dims=dims(), scale=0.0625, batch=2, t_q=4, qn=FAKE, qp=FAKE, wuk=FAKE, wuv=FAKE, kv=FAKE,
             dt=B.MLA_BF16, num_blocks=10, block_size=16, bt=FAKE, max_blocks=4, sl=FAKE, out=FAKE,
             out_dt=B.MLA_BF16, lse=None, ws=FAKE, ws_bytes=1 << 34, stream=None)
    a.update(kw)
    return mla.lib().mla_prefill_attention(a["dims"], a["scale"], a["batch"], a["t_q"], a["qn"], a["qp"], a["wuk"],
                                           a["wuv"], a["kv"], a["dt"], a["num_blocks"], a["block_size"], a["bt"],
                                           a["max_blocks"], a["sl"], a["out"], a["out_dt"], a["lse"], a["ws"],
                                           a["ws_bytes"], a["stream"])


def test_prefill_host_validation():
    sz = ctypes.c_size_t()
    L = mla.lib()
    assert L.mla_prefill_workspace_size(dims(), 2, 4, 16, ctypes.byref(sz)) == B.MLA_OK
    # header + status, then K_nope and V for 2 x 64 heads x 64 rows
    assert sz.value >= 2 * 64 * 64 * (192 + 256) * 2
    assert L.mla_prefill_workspace_size(dims((64, 256, 0, 256, 512)), 1, 8, 16, ctypes.byref(sz)) == B.MLA_OK
    assert L.mla_prefill_workspace_size(dims((4, 16, 8, 16, 32)), 1, 8, 16, ctypes.byref(sz)) == B.MLA_ERR_UNSUPPORTED
    assert L.mla_prefill_workspace_size(None, 1, 8, 16, ctypes.byref(sz)) == B.MLA_ERR_NULL
    assert L.mla_prefill_workspace_size(dims(), -1, 8, 16, ctypes.byref(sz)) == B.MLA_ERR_SHAPE
    assert L.mla_prefill_workspace_size(dims(), 1, 0, 16, ctypes.byref(sz)) == B.MLA_ERR_SHAPE
    assert L.mla_prefill_workspace_size(dims(), 1, 8, 32, ctypes.byref(sz)) == B.MLA_ERR_UNSUPPORTED
    assert prefill(dims=None) == B.MLA_ERR_NULL
    assert prefill(dims=dims((0, 192, 64, 256, 512))) == B.MLA_ERR_DIMS
    assert prefill(dims=dims((64, 128, 64, 256, 512))) == B.MLA_ERR_UNSUPPORTED   # qk width 192
    assert prefill(dims=dims((64, 192, 64, 128, 512))) == B.MLA_ERR_UNSUPPORTED   # d_v 128
    assert prefill(batch=-1) == B.MLA_ERR_SHAPE
    assert prefill(t_q=0) == B.MLA_ERR_SHAPE
    assert prefill(num_blocks=0) == B.MLA_ERR_SHAPE
    assert prefill(block_size=8) == B.MLA_ERR_UNSUPPORTED
    assert prefill(dt=B.MLA_F32) == B.MLA_ERR_UNSUPPORTED
    assert prefill(dt=3) == B.MLA_ERR_ARG
    assert prefill(scale=0.0) == B.MLA_ERR_ARG
    assert prefill(scale=math.nan) == B.MLA_ERR_ARG
    assert prefill(ws=None) == B.MLA_ERR_NULL
    assert prefill(ws_bytes=1024) == B.MLA_ERR_WORKSPACE
    assert prefill(qn=None) == B.MLA_ERR_NULL
    assert prefill(qp=None) == B.MLA_ERR_NULL   # rope part needed
    assert prefill(kv=None) == B.MLA_ERR_NULL
    assert prefill(out=None) == B.MLA_ERR_NULL
    assert prefill(batch=0, qn=None, qp=None, kv=None, out=None) == B.MLA_OK


def test_default_scale_and_strings():
    assert mla.mla_default_scale(GLM52) == pytest.approx(1 / 16, abs=1e-9)
    assert mla.mla_default_scale((64, 256, 0, 256, 512)) == pytest.approx(1 / 16, abs=1e-9)
    assert mla.mla_default_scale((4, 16, 8, 16, 32)) == pytest.approx(1 / math.sqrt(24), rel=1e-7)
    assert math.isnan(mla.lib().mla_default_scale(None))
    for code in range(8):
        assert len(mla.mla_status_string(code)) > 0
    assert mla.mla_status_string(99) == "unknown status"


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 64, 192, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mla.mla_absorb_q(GLM52, x, torch.zeros(4, 64, 64, dtype=torch.bfloat16),
                         torch.zeros(64, 192, 512, dtype=torch.bfloat16),
                         torch.zeros(4, 64, 576, dtype=torch.bfloat16))


def test_dcp_and_combine_host_validation():
    # Argument errors are reported before any device work (no GPU needed).
    L = mla.lib()
    fake = ctypes.c_void_p(0x1000)
    dims = mla.as_dims(GLM52)

    def dcp(world=2, rank=0, interleave=1, lse=fake, batch=2):
        return L.mla_decode_attention_dcp(ctypes.byref(dims), 0.0625, batch, 1, fake, fake, B.MLA_BF16, 64, 16,
                                          fake, 8, fake, world, rank, interleave, fake, B.MLA_F32, lse, fake,
                                          1 << 20, 0, None)
    assert dcp(world=0) == B.MLA_ERR_ARG
    assert dcp(rank=-1) == B.MLA_ERR_ARG
    assert dcp(rank=2) == B.MLA_ERR_ARG
    assert dcp(interleave=0) == B.MLA_ERR_ARG
    assert dcp(lse=None) == B.MLA_ERR_NULL

    def comb(width=512, n_rows=4, n_parts=2, o=fake, l=fake, out=fake, dt=B.MLA_F32):
        return L.mla_lse_combine(width, n_rows, n_parts, o, l, out, dt, None, None)
    assert comb(width=0) == B.MLA_ERR_SHAPE
    assert comb(n_rows=-1) == B.MLA_ERR_SHAPE
    assert comb(n_parts=0) == B.MLA_ERR_SHAPE
    assert comb(dt=5) == B.MLA_ERR_ARG
    assert comb(o=None) == B.MLA_ERR_NULL
    assert comb(l=None) == B.MLA_ERR_NULL
    assert comb(out=None) == B.MLA_ERR_NULL
    assert comb(n_rows=0, o=None, l=None, out=None) == B.MLA_OK


def test_noalloc_refuses_plans_beyond_its_scratch():
    # The allocation-free entry point's scratch holds 160 MiB; a plan that
    # needs more is refused before any device work (explicit range count: no
    # device query).
    L = mla.lib()
    dsv3 = (128, 128, 64, 0, 512)
    sz = ctypes.c_size_t()
    assert L.mla_decode_workspace_size(dims(dsv3), 64, 1, 2048, 16, 64, ctypes.byref(sz)) == B.MLA_OK
    assert sz.value > 160 << 20
    assert L.mla_decode_attention_noalloc(dims(dsv3), 0.07, 64, 1, FAKE, FAKE, B.MLA_BF16, 100000, 16, FAKE, 2048,
                                          FAKE, FAKE, B.MLA_BF16, None, 64, None) == B.MLA_ERR_WORKSPACE
    assert L.mla_decode_attention_noalloc(None, 0.07, 64, 1, FAKE, FAKE, B.MLA_BF16, 100000, 16, FAKE, 2048,
                                          FAKE, FAKE, B.MLA_BF16, None, 64, None) == B.MLA_ERR_NULL
