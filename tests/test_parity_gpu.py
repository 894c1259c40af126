"""HIP path vs the float64 oracle, element by element, on seeded inputs.

Sizes span several tiles and a ragged tail while the oracle still finishes in
seconds; the full-size workloads are checked on sampled channels, which the
oracle computes exactly because channels are independent.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from _helpers import DevInputs, compare, host64, run_gpu, run_oracle, sample_channels

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


W = synth.WORKLOADS


def _case(glr, wl, chunk=None, variant=0, chans=None, with_dh_last=False, force_reset0=False, label=""):
    inp = synth.make_inputs(wl, variant=variant, with_dh_last=with_dh_last, force_reset0=force_reset0)
    d = DevInputs(inp)
    gpu = run_gpu(glr, d, chunk=chunk)
    ref = run_oracle(inp, chans=chans)
    return compare(wl.io, gpu, ref, chans=chans, label=label or wl.name)


# ------------------------------------------------------------------ tiny f32 workload

@pytest.mark.parametrize("chunk", [0, 8, 16, 32, 64, 128, 256])
def test_tiny_f32_all_chunks(gpu_lib, chunk):
    _case(gpu_lib, W[0], chunk=chunk)


def test_tiny_f32_with_state_resets_and_final_grad(gpu_lib):
    wl = W[0].resized(batch=3, length=77, width=64)
    wl = synth.dataclasses.replace(wl, doc_mean=9.0, h0=True)
    _case(gpu_lib, wl, chunk=16, with_dh_last=True)


# ------------------------------------------------------------------ reduced bf16 workloads

@pytest.mark.parametrize("chunk", [0, 32, 128])
def test_restricted_reduced(gpu_lib, chunk):
    # restricted protocol: zero initial state, no resets; ragged length
    _case(gpu_lib, W[1].resized(batch=2, length=300, width=1024), chunk=chunk)


@pytest.mark.parametrize("width", [1, 3, 63, 65, 100, 130, 2560])
def test_ragged_widths(gpu_lib, width):
    wl = synth.dataclasses.replace(W[2].resized(batch=2, length=45, width=width), doc_mean=11.0)
    _case(gpu_lib, wl, chunk=16, with_dh_last=True)


@pytest.mark.parametrize("length", [1, 2, 7, 8, 9, 63, 64, 65])
def test_short_lengths(gpu_lib, length):
    wl = synth.dataclasses.replace(W[2].resized(batch=3, length=length, width=256), doc_mean=5.0)
    _case(gpu_lib, wl, chunk=32, with_dh_last=True)


def test_canonical_reset_reduced(gpu_lib):
    _case(gpu_lib, W[2].resized(batch=2, length=1500, width=512))


def test_canonical_dense_resets(gpu_lib):
    wl = synth.dataclasses.replace(W[2].resized(batch=4, length=600, width=256), doc_mean=20.0)
    _case(gpu_lib, wl, chunk=64, with_dh_last=True)


@pytest.mark.parametrize("length", [2048, 2048 + 37])
def test_long_memory_reduced(gpu_lib, length):
    # chunks of 256 with a partial last chunk, long-memory decay range
    _case(gpu_lib, W[3].resized(length=length, width=256))


def test_reset_at_t0_zeroes_dh0_and_ignores_h0(gpu_lib):
    wl = W[2].resized(batch=2, length=100, width=256)
    inp = synth.make_inputs(wl, force_reset0=True)
    d = DevInputs(inp)
    gpu = run_gpu(gpu_lib, d, chunk=16)
    assert torch.all(gpu["dh0"] == 0)
    d.h0 = d.h0 * 3.0 + 1.0
    gpu2 = run_gpu(gpu_lib, d, chunk=16)
    assert torch.equal(gpu["h"], gpu2["h"])
    compare(wl.io, gpu, run_oracle(inp))


# ------------------------------------------------------------------ randomised small shapes

def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    io = ("f32", "bf16")[seed % 2]
    B = int(rng.integers(1, 4))
    L = int(rng.choice([1, 2, 7, 8, 9, 63, 64, 65, 257, int(rng.integers(10, 600)), int(rng.integers(600, 2000))]))
    Wd = int(rng.choice([1, 2, 5, 64, 96, 127, 129, 200, int(rng.integers(1, 700))]))
    chunk = int(rng.choice([0, 8, 16, 32, 64, 128, 256]))
    doc = None if rng.random() < 0.3 else float(rng.choice([1.0, 3.0, 40.0, 500.0]))
    lo = float(rng.choice([1e-3, 0.5, 0.9, 0.99]))
    wl = synth.dataclasses.replace(W[2].resized(batch=B, length=L, width=Wd), io=io, doc_mean=doc,
                                   h0=bool(rng.random() < 0.5), decay_lo=lo, decay_hi=min(0.9999, lo + 0.099))
    return wl, chunk, bool(rng.random() < 0.5)


@pytest.mark.parametrize("seed", range(24))
def test_random_small_shapes(gpu_lib, seed):
    # shapes, chunk lengths, io types, reset densities, decay ranges and the
    # optional inputs drawn at random (fixed seeds), every case against the
    # oracle on all channels
    wl, chunk, dh_last = _random_case(seed)
    _case(gpu_lib, wl, chunk=chunk, variant=seed, with_dh_last=dh_last,
          label=f"seed {seed}: B={wl.batch} L={wl.length} W={wl.width} {wl.io} chunk {chunk} "
                f"docs {wl.doc_mean} h0 {wl.h0} decays [{wl.decay_lo}, {wl.decay_hi}]")


# ------------------------------------------------------------------ decay regimes and extreme logits

@pytest.mark.parametrize("io,lo,hi", [("f32", 0.01, 0.999), ("bf16", 0.01, 0.999), ("f32", 1e-6, 0.5)])
def test_wide_decay_range(gpu_lib, io, lo, hi):
    # per-step decays a = u^r with u = exp(-8 softplus(lambda)) ~ U[lo, hi] fall
    # on both sides of 0.9, where the kernels switch from the series for
    # 1 - a to 1 - a itself; the default workloads keep every a above 0.9
    wl = synth.dataclasses.replace(W[2].resized(batch=2, length=700, width=320), io=io, decay_lo=lo, decay_hi=hi)
    _case(gpu_lib, wl, label=f"decays U[{lo}, {hi}] {io}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_extreme_gate_logits(gpu_lib, io):
    # logits far enough out that the float32 sigmoid saturates to exactly 0
    # or 1: r = 0 gives a = 1 and 1 - a^2 = 0, where the backward's 1/m must
    # not turn into inf * 0; the float64 oracle stays finite down to -700
    wl = synth.dataclasses.replace(W[2].resized(batch=2, length=300, width=256), io=io)
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(7)
    extremes = np.array([-600.0, -200.0, -100.0, -89.0, -88.0, -87.0, -86.0, -80.0, -40.0, -20.0,
                         20.0, 40.0, 80.0, 100.0, 200.0, 600.0])
    for name in ("gx", "ga"):
        v = getattr(inp, name).value.copy()
        mask = rng.random(v.shape) < 0.3
        v[mask] = rng.choice(extremes, size=int(mask.sum()))
        setattr(inp, name, synth.store(v, io))
    d = DevInputs(inp)
    gpu = run_gpu(gpu_lib, d)
    for k in ("h", "dx", "dgx", "dga", "dlam", "dh0"):
        assert torch.isfinite(gpu[k]).all(), k
    ref = run_oracle(inp)
    compare(io, gpu, ref, label=f"extreme logits {io}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_extreme_decay_parameters(gpu_lib, io):
    # lambda far out on both sides: softplus(lambda) underflows (a = 1 at
    # every step, m = 0: the state never moves from h0) or is large enough
    # that a underflows to 0 (m = 1: the state is the latest write)
    wl = synth.dataclasses.replace(W[2].resized(batch=2, length=260, width=192), io=io)
    inp = synth.make_inputs(wl)
    vals = np.array([-200.0, -100.0, -90.0, -60.0, -30.0, -12.0, 12.0, 30.0, 80.0, 200.0], dtype=np.float32)
    idx = np.arange(0, wl.width, 7)[: 3 * len(vals)]
    lam = inp.lam.copy()
    lam[idx] = np.resize(vals, idx.size)
    inp.lam = lam
    gpu = run_gpu(gpu_lib, DevInputs(inp))
    for k in ("h", "dx", "dgx", "dga", "dlam", "dh0"):
        assert torch.isfinite(gpu[k]).all(), k
    compare(io, gpu, run_oracle(inp), label=f"extreme lambda {io}")


# ------------------------------------------------------------------ full sizes, sampled channels

@pytest.mark.parametrize("wid", [1, 2])
def test_full_size_pages_shape(gpu_lib, wid):
    wl = W[wid]
    ch = sample_channels(wl.width)
    _case(gpu_lib, wl, chans=ch)


@pytest.mark.parametrize("chunk", [8, 16, 32])
def test_full_size_short_chunks(gpu_lib, chunk):
    # shorter forward tiles run several workgroups per CU, which take every
    # tile from the ticket counter (a look-back must never wait on a tile of a
    # workgroup that has not started); no wait may reach its spin limit
    wl = W[1]
    ch = sample_channels(wl.width, n=16)
    _case(gpu_lib, wl, chunk=chunk, chans=ch, label=f"{wl.name} chunk {chunk}")
    assert max(ws.error_bits() for ws in gpu_lib.ops._default_ws.values()) == 0


@pytest.mark.parametrize("length", [32768, 32768 + 37])
def test_full_size_long_sequence(gpu_lib, length):
    wl = W[3].resized(length=length)
    ch = sample_channels(wl.width, n=24)
    _case(gpu_lib, wl, chans=ch)


def test_full_size_blockdiag_workload_scan(gpu_lib):
    # the scan of the 8 x 4096 x 2560 workload, on its own inputs as logits
    wl = W[4]
    ch = sample_channels(wl.width, n=24)
    _case(gpu_lib, wl, chans=ch)
