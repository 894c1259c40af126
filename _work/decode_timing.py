"""Times decode-sized forward calls (L = 1 and 8, h0 in, h_last out) through the
binding, for kernel traces of the latency-bound regime:

    rocprofv3 --kernel-trace --stats -d <dir> -o run -- python3 -u -m gated_linear_recurrence_amd.decode_timing

Prints the event-timed median per call for each shape (host-bound at these
sizes: the trace gives the kernel times).
"""
from __future__ import annotations

import numpy as np
import torch

import gated_linear_recurrence_amd as glr

SHAPES = ((1, 1, 2048), (4, 1, 2048), (16, 1, 4096), (4, 8, 2048), (4, 9, 2048))


def _median_us(fn, n=200, warm=20):
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3


def main():
    glr.load_library()
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for B, L, W in SHAPES:
        x, gx, ga = (torch.randn((B, L, W), device=dev, generator=g).to(torch.bfloat16) for _ in range(3))
        u = torch.empty(W, device=dev).uniform_(0.9, 0.999, generator=g)
        lam = torch.log(torch.expm1(-torch.log(u) / 8)).float()
        h0 = torch.randn((B, W), device=dev, generator=g)
        h = torch.empty_like(x)
        ws = glr.Workspace(dev)
        us = _median_us(lambda i: glr.rglru_fwd(x, gx, ga, lam, None, h0, h=h, training=False, want_h_last=True,
                                                workspace=ws))
        print(f"B={B} L={L} W={W}: {us:.2f} us per call (event-timed, host included)", flush=True)


if __name__ == "__main__":
    main()
