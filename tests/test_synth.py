"""The seeded input generators: reproducible draws, the target distributions, bf16 RNE storage."""
import math

import numpy as np
import torch

import synth


def test_draws_are_reproducible_and_distinct():
    wl = synth.WORKLOADS[0]
    a = synth.make_inputs(wl)
    b = synth.make_inputs(wl)
    np.testing.assert_array_equal(a.x.raw, b.x.raw)
    np.testing.assert_array_equal(a.lam, b.lam)
    assert not np.array_equal(a.x.raw, a.gx.raw)
    c = synth.make_inputs(wl, variant=1)
    assert not np.array_equal(a.x.raw, c.x.raw)


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                                  np.inf, -np.inf, 3.4e38], dtype=np.float32)])
    bits = synth.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    # ties go to even mantissa
    assert synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.float32([1.0 + 2 ** -8])))[0] == 1.0
    assert synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.float32([1.0 + 3 * 2 ** -8])))[0] == 1.0 + 2 ** -6
    nan_bits = synth.f32_to_bf16_bits(np.float32([np.nan]))
    assert np.isnan(synth.bf16_bits_to_f32(nan_bits))[0]


def test_stored_value_is_exact_value_of_storage():
    wl = synth.WORKLOADS[1].resized(batch=1, length=8, width=16)
    inp = synth.make_inputs(wl)
    np.testing.assert_array_equal(inp.x.value, synth.bf16_bits_to_f32(inp.x.raw).astype(np.float64))


def test_decay_parameter_hits_target_range():
    for wid, (lo, hi) in ((0, (0.9, 0.999)), (3, (0.99, 0.9999))):
        lam = synth.decay_param(wid, 20000, lo, hi).astype(np.float64)
        u = np.exp(-8.0 * np.logaddexp(0.0, lam))
        assert u.min() >= lo - 1e-6 and u.max() <= hi + 1e-6
        # uniform on [lo, hi]: the mean sits in the middle
        assert abs(u.mean() - (lo + hi) / 2) < 4 * (hi - lo) / math.sqrt(12 * 20000)


def test_reset_layout_statistics():
    B, L, mean = 64, 4096, 512.0
    flags = synth.reset_flags(2, B, L, mean)
    assert flags.dtype == np.uint8 and flags.shape == (B, L)
    assert set(np.unique(flags)) <= {0, 1}
    gaps = []
    firsts = []
    for b in range(B):
        pos = np.flatnonzero(flags[b])
        if len(pos):
            firsts.append(pos[0])
            gaps.extend(np.diff(pos))
    assert min(firsts) >= 1                         # t = 0 continues the carried-in document
    gaps = np.array(gaps)
    # Geometric(1/mean) on {1, 2, ...}: mean `mean`, std sqrt(1-p)/p
    p = 1.0 / mean
    sd = math.sqrt(1 - p) / p
    assert abs(gaps.mean() - mean) < 5 * sd / math.sqrt(len(gaps))


def test_workload_table_matches_the_stated_shapes():
    w = synth.WORKLOADS
    assert (w[0].batch, w[0].length, w[0].width, w[0].io) == (1, 64, 64, "f32")
    assert (w[1].batch, w[1].length, w[1].width, w[1].io, w[1].doc_mean, w[1].h0) == (4, 2048, 2048, "bf16", None, False)
    assert (w[2].doc_mean, w[2].h0) == (512.0, True)
    assert (w[3].batch, w[3].length, w[3].width, w[3].chunk, w[3].doc_mean) == (1, 32768, 4096, 256, 4096.0)
    assert (w[4].batch, w[4].length, w[4].width, w[4].proj_blocks, w[4].proj_block) == (8, 4096, 2560, 10, 256)
    assert (w[5].batch, w[5].length, w[5].width, w[5].doc_mean, w[5].h0, w[5].proj_blocks) == (4, 2048, 2048, None, False, 8)


def test_projection_weights_scale():
    wl = synth.WORKLOADS[4].resized(batch=1, length=4)
    inp = synth.make_inputs(wl)
    assert inp.wx.shape == (10, 256, 256)
    assert abs(inp.wx.value.std() - 1 / 16) < 0.002
    assert np.all(inp.bx.value == 0)


def test_delta_inputs_are_seeded_and_shaped():
    from synth import delta as sd
    wl = sd.DELTA_WORKLOADS[11].resized(batch=2, length=9, k_heads=1, v_heads=2, k_dim=16, v_dim=8, h0=True)
    a, b = sd.make_delta_inputs(wl), sd.make_delta_inputs(wl)
    for x, y in ((a.q.raw, b.q.raw), (a.k.raw, b.k.raw), (a.v.raw, b.v.raw), (a.g, b.g), (a.beta, b.beta), (a.h0, b.h0)):
        np.testing.assert_array_equal(x, y)
    assert a.q.shape == (2, 9, 1, 16) and a.v.shape == (2, 9, 2, 8) and a.g.shape == (2, 9, 2, 16)
    assert a.h0.shape == (2, 2, 16, 8)
    np.testing.assert_allclose(np.linalg.norm(a.k.value, axis=-1), 1.0, atol=1e-2)   # unit keys up to bf16 rounding
    assert np.all(a.g < 0) and np.all(np.exp(a.g) >= 0.9 - 1e-6) and np.all((a.beta > 0) & (a.beta < 1))
    p = sd.make_delta_inputs(wl.resized(kda=False), lengths=[3, 0, 5])
    assert p.cu.tolist() == [0, 3, 3, 8] and p.q.shape == (1, 8, 1, 16) and p.h0.shape == (3, 2, 16, 8)
    assert p.g.shape == (1, 8, 2)
