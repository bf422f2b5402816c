"""Pins of oracle.prolog, the fused MLA prolog of the CANN aclnnMlaProlog page
(its four paths: c^Q = RmsNorm(x W^DQ), q^N = c^Q W^UQ W^UK, q^R =
ROPE(c^Q W^QR), cache rows RmsNorm(x W^DKV) | ROPE(x W^KR)), against
properties of those formulas and an independent recomputation."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle

D3 = oracle.Dims(3, 8, 4, 0, 16)   # n_head, d_nope, d_rope, d_v, kv_rank
HID, QR = 24, 12


def draw(seed, n=5, hidden=HID, q_rank=QR, d=D3):
    rng = np.random.default_rng(seed)
    H, dn, dr, R = d.n_head, d.d_nope, d.d_rope, d.kv_rank
    w = dict(x=rng.standard_normal((n, hidden)), w_dq=rng.standard_normal((q_rank, hidden)) / np.sqrt(hidden),
             w_uq=rng.standard_normal((H * dn, q_rank)) / np.sqrt(q_rank),
             w_qr=rng.standard_normal((H * dr, q_rank)) / np.sqrt(q_rank),
             w_uk=rng.standard_normal((H, dn, R)) / np.sqrt(dn), w_dkv=rng.standard_normal((R, hidden)) / np.sqrt(hidden),
             w_kr=rng.standard_normal((dr, hidden)) / np.sqrt(hidden), gamma_q=1 + 0.1 * rng.standard_normal(q_rank),
             gamma_kv=1 + 0.1 * rng.standard_normal(R))
    w["positions"] = rng.integers(0, 5000, n).astype(np.int32)
    w["slots"] = rng.permutation(2 * n)[:n].astype(np.int64)
    return w


def run(w, d=D3, eps=(1e-6, 1e-6), style=oracle.NEOX, base=1e4, num_slots=None):
    n = w["x"].shape[0]
    cache = np.zeros((num_slots or 2 * n, d.kv_rank + d.d_rope))
    q, bad = oracle.prolog(d, w["x"], w["w_dq"], w["w_uq"], w["w_qr"], w["w_uk"], w["w_dkv"], w["w_kr"],
                           w["gamma_q"], w["gamma_kv"], eps[0], eps[1], w["positions"], base, style, w["slots"], cache)
    assert bad == 0
    return q, cache


def test_input_scale_is_removed_by_both_norms():
    # RmsNorm(a y) = RmsNorm(y) for a > 0 when eps = 0: q^N, q^R and the
    # latent cache rows do not change; k^R is not normalised and scales by a.
    w = draw(1)
    q1, c1 = run(w, eps=(0.0, 0.0))
    w2 = dict(w, x=w["x"] * 7.5)
    q2, c2 = run(w2, eps=(0.0, 0.0))
    R = D3.kv_rank
    np.testing.assert_allclose(q2, q1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c2[:, :R], c1[:, :R], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c2[:, R:], 7.5 * c1[:, R:], rtol=1e-12, atol=1e-12)


def test_position_zero_leaves_rope_parts_unrotated():
    w = draw(2)
    w["positions"][:] = 0
    q, c = run(w)
    H, dn, dr, R = D3.n_head, D3.d_nope, D3.d_rope, D3.kv_rank
    x = w["x"]
    cq_pre = x @ w["w_dq"].T
    cq = w["gamma_q"] * cq_pre / np.sqrt(np.mean(cq_pre ** 2, axis=1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(q[:, :, R:], (cq @ w["w_qr"].T).reshape(-1, H, dr), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c[w["slots"], R:], x @ w["w_kr"].T, rtol=1e-12, atol=1e-12)


def test_each_weight_scales_only_its_path():
    w = draw(3)
    q1, c1 = run(w)
    R = D3.kv_rank
    qa, _ = run(dict(w, w_uq=2 * w["w_uq"]))     # q^N doubles, q^R unchanged
    np.testing.assert_allclose(qa[:, :, :R], 2 * q1[:, :, :R], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(qa[:, :, R:], q1[:, :, R:], rtol=1e-12, atol=1e-12)
    qb, _ = run(dict(w, w_qr=-3 * w["w_qr"]))    # q^R scales, q^N unchanged
    np.testing.assert_allclose(qb[:, :, R:], -3 * q1[:, :, R:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(qb[:, :, :R], q1[:, :, :R], rtol=1e-12, atol=1e-12)
    _, cb = run(dict(w, w_kr=2 * w["w_kr"]))     # only the cache's rope part
    np.testing.assert_allclose(cb[:, R:], 2 * c1[:, R:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(cb[:, :R], c1[:, :R], rtol=1e-12, atol=1e-12)


def test_head_permutation_permutes_outputs():
    w = draw(4)
    H, dn, dr = D3.n_head, D3.d_nope, D3.d_rope
    perm = np.array([2, 0, 1])
    wp = dict(w, w_uq=w["w_uq"].reshape(H, dn, -1)[perm].reshape(H * dn, -1),
              w_qr=w["w_qr"].reshape(H, dr, -1)[perm].reshape(H * dr, -1), w_uk=w["w_uk"][perm])
    q1, _ = run(w)
    q2, _ = run(wp)
    np.testing.assert_allclose(q2, q1[:, perm], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("style", [oracle.NEOX, oracle.INTERLEAVED])
def test_against_independent_recomputation(style):
    # torch for the products and the norms, numpy complex numbers for the
    # rotation, einsum for the absorb; a bf16-stored input set.
    spec = mi.with_spec(mi.SPECS["glm52_decode"], dtype="bf16")
    w = draw(5, n=4)
    for k in ("x", "w_dq", "w_uq", "w_qr", "w_uk", "w_dkv", "w_kr"):
        w[k] = mi.store(w[k], spec.dtype)  # bf16 bit patterns
    q, c = run(w, style=style, base=8e6)
    f = lambda a: torch.from_numpy(mi.widen(a).astype(np.float64))
    H, dn, dr, R = D3.n_head, D3.d_nope, D3.d_rope, D3.kv_rank
    x = f(w["x"])
    g_q, g_kv = torch.from_numpy(w["gamma_q"]), torch.from_numpy(w["gamma_kv"])
    cq = torch.nn.functional.rms_norm(x @ f(w["w_dq"]).T, (QR,), g_q, 1e-6)
    qn = torch.einsum("nhp,hpl->nhl", (cq @ f(w["w_uq"]).T).reshape(-1, H, dn), f(w["w_uk"]))

    def rot(v, pos):  # v [..., dr] rotated at per-row positions, by complex multiplication
        v = v.numpy()
        half = dr // 2
        inv = 8e6 ** (-2.0 * np.arange(half) / dr)
        ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]
        ph = np.exp(1j * ang)
        if style == oracle.NEOX:
            z = (v[..., :half] + 1j * v[..., half:]) * ph.reshape(ph.shape[0], *([1] * (v.ndim - 2)), half)
            return np.concatenate([z.real, z.imag], axis=-1)
        z = (v[..., 0::2] + 1j * v[..., 1::2]) * ph.reshape(ph.shape[0], *([1] * (v.ndim - 2)), half)
        out = np.empty_like(v)
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
        return out
    qr = rot((cq @ f(w["w_qr"]).T).reshape(-1, H, dr), w["positions"])
    np.testing.assert_allclose(q[:, :, :R], qn.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(q[:, :, R:], qr, rtol=1e-10, atol=1e-10)
    ckv = torch.nn.functional.rms_norm(x @ f(w["w_dkv"]).T, (R,), g_kv, 1e-6).numpy()
    kr = rot(x @ f(w["w_kr"]).T, w["positions"])
    np.testing.assert_allclose(c[w["slots"], :R], ckv, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(c[w["slots"], R:], kr, rtol=1e-10, atol=1e-10)


def test_identity_down_projection_normalises_the_input():
    # hidden == q_rank and W^DQ = I, gamma 1, eps 0: c^Q = x / rms(x), so with
    # W^UQ = I on one head and W^UK = I the latent query is x / rms(x).
    d = oracle.Dims(1, 6, 2, 0, 6)
    w = draw(6, n=3, hidden=6, q_rank=6, d=d)
    w.update(w_dq=np.eye(6), w_uq=np.eye(6), w_uk=np.eye(6)[None], gamma_q=np.ones(6))
    q, _ = run(w, d=d, eps=(0.0, 1e-6))
    x = w["x"]
    np.testing.assert_allclose(q[:, 0, :6], x / np.sqrt(np.mean(x * x, axis=1, keepdims=True)), rtol=1e-13, atol=1e-13)
