"""HIP-graph replay of the decode step (as the benchmark runs it): every replay, with eager
work and synchronisations in between, matches the eager result bit for bit, and the
eager result matches the oracle."""
import numpy as np
import pytest
import torch

import bitlinear_fwd_amd as bl
import oracle
from bitlinear_fwd_amd import synth
from gpu_helpers import acts_host_f32, check_equal, check_y, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_graph_replays_match_eager():
    print("case: graph replay of fused decode + two-kernel decode + prefill", flush=True)
    shapes = [(1, 2560, 6912), (1, 6912, 2560), (8, 640, 2560), (40, 300, 512)]
    mats = []
    for i, (m, k, n) in enumerate(shapes):
        w = synth.latent_weights(n, k, seed=9100 + i, device=DEV)
        packed, gamma = bl.quantize_weights(w)
        x = synth.activations(m, k, seed=9600 + i, dtype=torch.bfloat16, device=DEV)
        xq = torch.empty((m, bl.k_pad(k)), dtype=torch.int8, device=DEV)
        a = torch.empty(m, dtype=torch.float32, device=DEV)
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        mats.append(dict(m=m, k=k, n=n, packed=packed, gamma=gamma, x=x, xq=xq, a=a, y=y))

    def step():
        for d in mats:
            if d["m"] <= 4:
                bl.forward_fused(d["packed"], d["gamma"], d["x"], d["n"], d["k"], y=d["y"], xq=d["xq"], absmax=d["a"])
            else:
                bl.quantize_acts(d["x"], d["xq"], d["a"])
                bl.forward(d["packed"], d["gamma"], d["xq"], d["a"], d["n"], d["k"], y=d["y"])

    step()
    torch.cuda.synchronize()
    eager = [d["y"].clone() for d in mats]
    # the eager result is the oracle's
    for d, ye in zip(mats, eager):
        xq_ref, a_ref = oracle.quant_acts(acts_host_f32(d["x"]))
        q = oracle.unpack(host(d["packed"]), d["n"], d["k"])
        _, y_ref = oracle.forward(q, np.float32(host(d["gamma"])[0]), xq_ref, a_ref, d["k"])
        check_y(host(ye), y_ref, f"eager {d['m']}x{d['k']}x{d['n']}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(5):
        for d in mats:
            d["y"].fill_(float("nan"))
            d["xq"].fill_(0)
        scratch = torch.randn(1 << 20, device=DEV).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for d, ye in zip(mats, eager):
            check_equal(host(d["y"]).view(np.uint32), host(ye).view(np.uint32), f"replay {rep}")
