"""Gated delta rule entry points captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A decode step (the forward of one token per sequence from a nonzero state),
a training step (the forward writing its checkpoint, then the backward) and
the GDN chunk form on packed sequences are captured once and replayed
several times. Between replays an eager call
on other inputs overwrites the same outputs, checkpoint and workspace, so a
replay only matches if the captured kernels rewrite everything they read.
Every replay must equal the eager results bitwise; the kernels clear no
memory with memset nodes (the backward's partial sums are written in full
before the reduce reads them).
"""
import sys

import numpy as np
import pytest
import torch

from synth import delta as sd

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def _dev(stored):
    t = torch.from_numpy(stored.raw.copy()).cuda()
    return t.view(torch.bfloat16) if stored.io == "bf16" else t


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _inputs(wl, variant):
    inp = sd.make_delta_inputs(wl, variant=variant)
    d = {"q": _dev(inp.q), "k": _dev(inp.k), "v": _dev(inp.v), "g": _f32(inp.g), "beta": _f32(inp.beta),
         "h0": _f32(inp.h0)}
    rng = np.random.default_rng(1000 + variant)
    d["do"] = torch.from_numpy(rng.standard_normal(inp.v.value.shape).astype(np.float32)).cuda().to(d["v"].dtype)
    d["dhl"] = _f32(rng.standard_normal(inp.h0.shape))
    return d


def _replays_match(step, live, other, ref):
    """Capture step(live), then replay it three times, each after an eager step(other)."""
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step(live)  # warm-up on the capture stream, as torch recommends
    torch.cuda.current_stream().wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            outs = step(live)
    torch.cuda.synchronize()
    for r in range(3):
        step(other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(ref.keys(), outs, ref.values()):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager call"
    del graph


def test_decode_step_graph_replay(gpu_lib):
    glr = gpu_lib
    wl = sd.DELTA_WORKLOADS[12].resized(wid=50, batch=16, v_heads=4, k_heads=4)
    live, other = _inputs(wl, 1), _inputs(wl, 2)
    o = torch.empty_like(live["v"])
    fs = torch.empty_like(live["h0"])

    def step(d):
        glr.rglru_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"], o=o,
                                 final_state=fs)
        return o, fs

    step(live)
    torch.cuda.synchronize()
    ref = {"o": o.clone(), "final_state": fs.clone()}
    _replays_match(step, live, other, ref)


@pytest.mark.parametrize("kda", [False, True])
def test_training_step_graph_replay(gpu_lib, kda):
    glr = gpu_lib
    wl = sd.DELTA_WORKLOADS[10].resized(wid=51, batch=2, length=40, k_heads=1, v_heads=2, k_dim=64, v_dim=64,
                                        kda=kda, h0=True)
    live, other = _inputs(wl, 3), _inputs(wl, 4)
    o = torch.empty_like(live["v"])
    fs = torch.empty_like(live["h0"])
    shape = glr.ops._delta_common(live["q"], live["k"], live["v"], live["g"], live["beta"], None, live["h0"],
                                  None, False, True, o, fs)[0]
    ck = torch.empty(glr.rglru_delta_ckpt_elems(shape, 0), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(glr.rglru_delta_bwd_workspace_bytes(shape, 0), 1), dtype=torch.uint8, device="cuda")
    grads = [torch.empty_like(live["q"]), torch.empty_like(live["k"]), torch.empty_like(live["v"]),
             torch.empty_like(live["g"]), torch.empty_like(live["beta"]), torch.empty_like(live["h0"])]

    def step(d):
        glr.rglru_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"], o=o,
                                 final_state=fs, ckpt=ck)
        got = glr.rglru_delta_rule_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], ck, d["do"], d["dhl"],
                                       workspace=ws)
        for dst, src in zip(grads, got):
            dst.copy_(src)
        return (o, fs, *grads)

    step(live)
    torch.cuda.synchronize()
    names = ["o", "final_state", "dq", "dk", "dv", "dg", "dbeta", "dh0"]
    ref = {n: t.clone() for n, t in zip(names, (o, fs, *grads))}
    _replays_match(step, live, other, ref)


def test_chunk_form_graph_replay(gpu_lib):
    """The GDN chunk form on packed sequences (its chunk map is rebuilt on the device each call)."""
    glr = gpu_lib
    lens = [70, 0, 1, 130, 64]
    wl = sd.DELTA_WORKLOADS[10].resized(wid=52, k_heads=1, v_heads=2, k_dim=128, v_dim=64, h0=True)

    def inputs(variant):
        inp = sd.make_delta_inputs(wl, variant=variant, lengths=lens)
        return {"q": _dev(inp.q), "k": _dev(inp.k), "v": _dev(inp.v), "g": _f32(inp.g), "beta": _f32(inp.beta),
                "h0": _f32(inp.h0), "cu": torch.from_numpy(inp.cu).cuda()}

    live, other = inputs(5), inputs(6)
    o = torch.empty_like(live["v"])
    fs = torch.empty_like(live["h0"])
    shape = glr.ops._delta_common(live["q"], live["k"], live["v"], live["g"], live["beta"], None, live["h0"],
                                  live["cu"], False, True, o, fs)[0]
    ws = torch.empty(glr.rglru_delta_chunk_workspace_bytes(shape, len(lens)), dtype=torch.uint8, device="cuda")

    def step(d):
        glr.rglru_delta_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"],
                                  cu_seqlens=d["cu"], o=o, final_state=fs, workspace=ws)
        return o, fs

    step(live)
    torch.cuda.synchronize()
    ref = {"o": o.clone(), "final_state": fs.clone()}
    _replays_match(step, live, other, ref)
