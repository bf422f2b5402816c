"""The seeded input generator: determinism, rounding, layout."""
import numpy as np
import torch

import mla_inputs as mi


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895314e38, -3.3895314e38,
                  np.inf, -np.inf, 1e-40, -1e-40, 6e-39], np.float32),
        # exact ties between two bf16 values (round to even both ways)
        (mi.bf16_bits_to_f32(np.arange(0x3F80, 0x3FA0, dtype=np.uint16)).view(np.uint32)
         + np.uint32(0x8000)).view(np.float32),
    ])
    ours = mi.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    nan = mi.to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(mi.bf16_bits_to_f32(nan)).all()


def test_widen_is_exact():
    b = np.arange(0, 65536, dtype=np.uint16)
    f = mi.bf16_bits_to_f32(b)
    ok = ~np.isnan(f)
    np.testing.assert_array_equal(mi.to_bf16_bits(f[ok]), b[ok])


def test_streams_are_counter_based_and_deterministic():
    k = mi.tensor_key(202, "c_kv")
    a = mi.normals(k, 0, 1001)
    np.testing.assert_array_equal(mi.normals(k, 0, 1001), a)
    np.testing.assert_array_equal(mi.normals(k, 37, 500), a[37:537])
    np.testing.assert_array_equal(mi.normals(k, 38, 11), a[38:49])
    assert not np.array_equal(mi.normals(mi.tensor_key(202, "k_pe"), 0, 1001), a)
    x = mi.normals(k, 0, 400000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_case_layout():
    spec = mi.SPECS["tiny_f32"]
    c = mi.make_case(spec)
    assert c.kv.shape == (4 + 2, 16, 40)
    used = c.block_table[c.block_table >= 0]
    assert len(set(used.tolist())) == used.size == 4
    assert (c.block_table[0, 1:] == -1).all()
    # spare blocks and tail rows are NaN, live rows are finite
    live = np.zeros(c.kv.shape[:2], bool)
    for b, L in enumerate(c.seq_lens):
        for j in range(L):
            live[c.block_table[b, j // 16], j % 16] = True
    assert np.isfinite(c.kv[live]).all() and np.isnan(c.kv[~live]).all()
    # relabelling changes the table, not the logical rows
    c2 = mi.make_case(spec, relabel_seed=5)
    for b in range(2):
        for j in range(c.seq_lens[b]):
            np.testing.assert_array_equal(c.kv[c.block_table[b, j // 16], j % 16],
                                          c2.kv[c2.block_table[b, j // 16], j % 16])


def test_rms_normalised_rows():
    spec = mi.with_spec(mi.SPECS["glm52_decode"], batch=2, seq_len=20)
    rows = mi.logical_rows(spec, mi.seq_lens_for(spec), 1)
    ckv = rows[:, :512]
    rms = np.sqrt((ckv * ckv).mean(1))
    assert np.all(np.abs(rms - 1) < 0.01)


def test_ragged_lengths():
    spec = mi.SPECS["dsv3_ragged"]
    L = mi.seq_lens_for(spec)
    assert L.shape == (64,) and L[0] == 0 and L[63] == 0
    assert L.min() >= 0 and L.max() <= 32768
    assert len(set(L.tolist())) > 50
