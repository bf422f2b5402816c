"""Helpers for the GPU parity tests: move a generated case to the device, run
the hot path through the C ABI, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import mla_inputs as mi
import mla_latent_cache_amd as mla
import oracle

DEV = "cuda"

# Tolerances: float32 inputs, max abs diff 1e-4; bf16 inputs, elementwise
# |gpu - oracle| <= 2e-2 + 1e-2 |oracle| against an oracle fed the same
# bf16-rounded values, plus a stricter whole-tensor check
# max |gpu - oracle| <= 1e-2 max |oracle|.
F32_ATOL = 1e-4
BF16_ATOL, BF16_RTOL, BF16_MAXREL = 2e-2, 1e-2, 1e-2


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def dims_tuple(spec):
    return (spec.n_head, spec.d_nope, spec.d_rope, spec.d_v, spec.kv_rank)


def oracle_dims(spec):
    return oracle.Dims(spec.n_head, spec.d_nope, spec.d_rope, spec.d_v, spec.kv_rank)


def store_dtype(spec):
    return torch.float32 if spec.dtype == "f32" else torch.bfloat16


class DeviceCase:
    """Device copies of a case's inputs."""

    def __init__(self, case: mi.Case):
        self.case = case
        s = case.spec
        self.kv = to_dev(case.kv)
        self.bt = torch.from_numpy(case.block_table).to(DEV)
        self.sl = torch.from_numpy(case.seq_lens).to(DEV)
        if s.q_given:
            self.q_abs_in = to_dev(case.q_abs)
        else:
            self.q_nope = to_dev(case.q_nope)
            self.q_pe = to_dev(case.q_pe) if s.d_rope else None
            self.w_uk = to_dev(case.w_uk)
            self.w_uv = to_dev(case.w_uv)


def run(dc: DeviceCase, num_splits: int = 0, out_dtype=None, with_lse: bool = True,
        decompress: bool = True, seq_lens=None, block_table=None):
    """Run absorb (unless the queries are given) -> decode -> decompress."""
    case, s = dc.case, dc.case.spec
    dims = dims_tuple(s)
    B, T, H, D, R = s.batch, s.t_q, s.n_head, s.D, s.kv_rank
    odt = out_dtype or store_dtype(s)
    if s.q_given:
        q_abs = dc.q_abs_in
    else:
        q_abs = torch.empty(B, T, H, D, dtype=store_dtype(s), device=DEV)
        mla.mla_absorb_q(dims, dc.q_nope, dc.q_pe, dc.w_uk, q_abs)
    bt = dc.bt if block_table is None else block_table
    sl = dc.sl if seq_lens is None else seq_lens
    out_lat = torch.empty(B, T, H, R, dtype=odt, device=DEV)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=DEV) if with_lse else None
    ws = torch.empty(mla.mla_decode_workspace_size(dims, B, T, bt.shape[1], 16, num_splits),
                     dtype=torch.uint8, device=DEV)
    mla.mla_decode_attention(dims, case.scale, q_abs, dc.kv, bt, sl, out_lat, lse, ws, num_splits)
    out = None
    if decompress and not s.q_given:
        out = torch.empty(B * T, H, s.d_v, dtype=odt, device=DEV)
        mla.mla_decompress_v(dims, out_lat, dc.w_uv, out)
    torch.cuda.synchronize()
    status = mla.mla_decode_status(ws)
    return dict(q_abs=q_abs, o_lat=out_lat, lse=lse, out=out, status=status, ws=ws)


def assert_close(g, o, spec_dtype: str, what: str):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    assert np.isfinite(o).all(), f"{what}: oracle not finite"
    assert np.isfinite(g).all(), f"{what}: GPU output has non-finite values"
    err = np.abs(g - o)
    if spec_dtype == "f32":
        assert err.max() <= F32_ATOL, f"{what}: max abs diff {err.max():.3e} > {F32_ATOL}"
        return float(err.max())
    bound = BF16_ATOL + BF16_RTOL * np.abs(o)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements outside 2e-2 + 1e-2|ref| (max err {err.max():.3e})"
    scale = max(np.abs(o).max(), 1e-30)
    assert err.max() <= BF16_MAXREL * scale, f"{what}: max err {err.max():.3e} > 1e-2 * max|ref| {scale:.3e}"
    return float(err.max() / scale)


def assert_lse_close(g, o, spec_dtype: str, what: str):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    ninf = np.isneginf(o)
    assert np.array_equal(np.isneginf(g), ninf), f"{what}: -inf pattern differs"
    fin = ~ninf
    if fin.any():
        assert_close(g[fin], o[fin], spec_dtype, what)


def oracle_q_abs(case):
    """The oracle's own absorbed queries [B][t_q][H][D] (float64), or the given ones."""
    s = case.spec
    if s.q_given:
        return case.q_abs
    q = oracle.absorb(oracle_dims(s), case.q_nope, case.q_pe, case.w_uk)
    return q.reshape(s.batch, s.t_q, s.n_head, s.D)


def paged(case):
    return oracle.Paged(case.kv, case.block_table, case.seq_lens)


def flat_index(spec, sel):
    sel = np.asarray(sel)
    return (sel[:, 0] * spec.t_q + sel[:, 1]) * spec.n_head + sel[:, 2]
