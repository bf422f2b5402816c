"""Pins of the oracle's cache-append prolog: RmsNorm, rope of rows at
per-row positions, and the slot-mapped cache write.

Each check compares the oracle with something outside it: torch's rms_norm
(a library routine the oracle never calls), numpy complex rotation, closed
forms of special inputs, invariants of the definitions, and a brute-force
scatter rebuilt from those library results.  A dropped mean, epsilon outside
the root, a misapplied gamma, a position taken from the wrong row, a head
index error, a wrong pairing, a write to a skipped slot or an off-by-one row
width each fail one of them.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle


def _rows(key, n, w, scale_spread=True):
    x = mi.normals(key, 0, n * w).reshape(n, w)
    if scale_spread:
        x *= np.exp(mi.normals(key + 1, 0, n))[:, None]
    return x


# --------------------------------------------------------------------------
# RmsNorm
# --------------------------------------------------------------------------
def test_rmsnorm_rows_have_unit_mean_square():
    x = _rows(11, 7, 48)
    y = oracle.rmsnorm(x, None, 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=0, atol=1e-13)


def test_rmsnorm_constant_rows_closed_form():
    # All-equal rows a: RMS = sqrt(a^2 + eps).  a = 1, eps = 3 gives exactly 1/2
    # (a sum instead of a mean, or eps outside the root, gives another value).
    y = oracle.rmsnorm(np.ones((2, 40)), None, 3.0)
    np.testing.assert_array_equal(y, 0.5)
    y = oracle.rmsnorm(np.full((1, 9), -2.0), None, 0.0)
    np.testing.assert_array_equal(y, -1.0)
    y = oracle.rmsnorm(np.zeros((1, 5)), None, 1e-6)
    np.testing.assert_array_equal(y, 0.0)


def test_rmsnorm_scale_invariance_and_gamma():
    x = _rows(21, 5, 32)
    g = 1.0 + 0.1 * mi.normals(23, 0, 32)
    y1 = oracle.rmsnorm(x, None, 0.0)
    np.testing.assert_allclose(oracle.rmsnorm(x * 37.5, None, 0.0), y1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.rmsnorm(x, g, 0.0), y1 * g[None, :], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.25])
def test_rmsnorm_matches_torch_rms_norm(dtype, eps):
    x = mi.store(_rows(31, 9, 512), dtype)
    g = mi.store(1.0 + 0.1 * mi.normals(33, 0, 512), dtype)
    xt = torch.from_numpy(mi.widen(x).astype(np.float64))
    gt = torch.from_numpy(mi.widen(g).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (512,), weight=gt, eps=eps).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(x, g, eps), ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Rope of rows at per-row positions
# --------------------------------------------------------------------------
def _complex_rope(x, pos, base, style):
    """numpy complex rotation of x [n][h][d] by pos[n] * base^(-2j/d)."""
    n, h, d = x.shape
    th = np.asarray(pos, np.float64)[:, None] * base ** (-2.0 * np.arange(d // 2) / d)[None, :]
    rot = np.exp(1j * th)[:, None, :]
    out = np.empty_like(x)
    if style == oracle.NEOX:
        z = (x[..., :d // 2] + 1j * x[..., d // 2:]) * rot
        out[..., :d // 2], out[..., d // 2:] = z.real, z.imag
    else:
        z = (x[..., 0::2] + 1j * x[..., 1::2]) * rot
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


@pytest.mark.parametrize("style", [oracle.NEOX, oracle.INTERLEAVED])
def test_rope_rows_matches_complex_rotation(style):
    x = mi.normals(41, 0, 6 * 3 * 16).reshape(6, 3, 16)
    pos = np.array([0, 1, 17, 4096, 131071, 1000000], np.int32)
    y = oracle.rope_rows(x, pos, mi.ROPE_BASE, style)
    np.testing.assert_allclose(y, _complex_rope(x, pos, mi.ROPE_BASE, style), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(y[0], x[0])


def test_rope_rows_dot_depends_on_position_difference_only():
    x = mi.normals(51, 0, 4 * 2 * 64).reshape(4, 2, 64)
    yq = oracle.rope_rows(x, np.array([10, 500, 10, 90000], np.int32), mi.ROPE_BASE)
    yk = oracle.rope_rows(x[::-1].copy(), np.array([3, 493, 10, 89993], np.int32), mi.ROPE_BASE)
    d = [float(yq[r, h] @ yk[r, h]) for r in range(4) for h in range(2)]
    # Rows 0, 1 and 3 sit 7 positions apart: equal dots for equal inputs;
    # row 2 sits at the same position on both sides: the unrotated dot.
    x_rev = x[::-1]
    d7 = [float(oracle.rope_neox(x[r, h], 7, mi.ROPE_BASE) @ x_rev[r, h]) for r in range(4) for h in range(2)]
    for r in (0, 1, 3):
        for h in range(2):
            assert abs(d[2 * r + h] - d7[2 * r + h]) <= 1e-9 * max(1.0, abs(d7[2 * r + h]))
    for h in range(2):
        assert abs(d[4 + h] - float(x[2, h] @ x_rev[2, h])) <= 1e-9


# --------------------------------------------------------------------------
# Slot-mapped cache append
# --------------------------------------------------------------------------
@pytest.mark.parametrize("style", [oracle.NEOX, oracle.INTERLEAVED])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cache_append_brute_force(style, dtype):
    kv_rank, d_rope, num_slots, n_tok = 24, 8, 48, 20
    c = mi.store(_rows(61, n_tok, kv_rank), dtype)
    k = mi.store(mi.normals(63, 0, n_tok * d_rope).reshape(n_tok, d_rope), dtype)
    g = mi.store(1.0 + 0.1 * mi.normals(65, 0, kv_rank), dtype)
    pos = mi.random_positions(67, n_tok, 200000)
    slots = mi.random_slots(69, num_slots, n_tok, n_skip=4, n_out=3)
    before = mi.normals(71, 0, num_slots * (kv_rank + d_rope)).reshape(num_slots, kv_rank + d_rope)
    cache = before.copy()
    bad = oracle.cache_append(cache, kv_rank, c, k, g, 1e-6, pos, mi.ROPE_BASE, style, slots)
    assert bad == 3

    cw = torch.from_numpy(mi.widen(c).astype(np.float64))
    gw = torch.from_numpy(mi.widen(g).astype(np.float64))
    lat = torch.nn.functional.rms_norm(cw, (kv_rank,), weight=gw, eps=1e-6).numpy()
    rope = _complex_rope(mi.widen(k).astype(np.float64)[:, None, :], pos, mi.ROPE_BASE, style)[:, 0]
    expect = before.copy()
    for n in range(n_tok):
        s = int(slots[n])
        if 0 <= s < num_slots:
            expect[s, :kv_rank] = lat[n]
            expect[s, kv_rank:] = rope[n]
    written = sorted(int(s) for s in slots if 0 <= s < num_slots)
    untouched = [r for r in range(num_slots) if r not in written]
    np.testing.assert_array_equal(cache[untouched], before[untouched])
    np.testing.assert_allclose(cache, expect, rtol=1e-12, atol=1e-12)


def test_cache_append_without_rope_part_and_all_skipped():
    kv_rank, num_slots = 16, 8
    c = _rows(81, 3, kv_rank)
    cache = np.zeros((num_slots, kv_rank))
    assert oracle.cache_append(cache, kv_rank, c, None, None, 0.0, None, 1.0, oracle.NEOX,
                               np.array([5, -1, 0])) == 0
    np.testing.assert_allclose(np.mean(cache[[5, 0]] ** 2, axis=1), 1.0, atol=1e-13)
    assert not cache[[1, 2, 3, 4, 6, 7]].any()
    before = cache.copy()
    assert oracle.cache_append(cache, kv_rank, c, None, None, 0.0, None, 1.0, oracle.NEOX,
                               np.array([-1, -1, -5])) == 0
    np.testing.assert_array_equal(cache, before)


def test_step_append_slots_follow_the_block_table():
    spec = mi.with_spec(mi.SPECS["glm52_causal_tq4"], batch=3, max_blocks=8, seq_len=0,
                        fixed_lens=(37, 2, 16), spare_blocks=2)
    case = mi.make_case(spec, poison=False)
    ap = mi.step_append(spec, case.seq_lens, case.block_table, n_pad=2)
    assert ap.slots.shape == (3 * 4 + 2,)
    # Request 0 (37 rows): new rows 33..36; request 1 is shorter than t_q: padding.
    for i in range(4):
        p = 33 + i
        assert ap.positions[i] == p
        assert ap.slots[i] == case.block_table[0, p // 16] * 16 + p % 16
    assert (ap.slots[4:8] == -1).all() and (ap.slots[12:] == -1).all()
    assert list(ap.positions[8:12]) == [12, 13, 14, 15]
