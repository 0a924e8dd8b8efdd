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


def test_grouped_call_replays_in_a_graph():
    print("case: graph replay of a grouped call (gate + up) and the 9..16-token decode", flush=True)
    k = 2560
    mats = []
    for i, n in enumerate((6912, 6912)):
        w = synth.latent_weights(n, k, seed=9300 + i, device=DEV)
        packed, gamma = bl.quantize_weights(w)
        mats.append((packed, gamma, n))
    x = synth.activations(1, k, seed=9400, dtype=torch.bfloat16, device=DEV)
    x16 = synth.activations(16, k, seed=9401, dtype=torch.bfloat16, device=DEV)
    xq = torch.empty((1, bl.k_pad(k)), dtype=torch.int8, device=DEV)
    a = torch.empty(1, dtype=torch.float32, device=DEV)
    xq16 = torch.empty((16, bl.k_pad(k)), dtype=torch.int8, device=DEV)
    a16 = torch.empty(16, dtype=torch.float32, device=DEV)
    ys = [torch.empty((1, n), dtype=torch.float32, device=DEV) for _, _, n in mats]
    y16 = torch.empty((16, 6912), dtype=torch.float32, device=DEV)
    # a pre-marshalled call holds the stream current when it was prepared, so a graph
    # captures the binding's call (which takes the capture stream); eagerly both agree
    bl.prepare_forward_grouped([(p, g, n, y) for (p, g, n), y in zip(mats, ys)], x, k, xq, a)()
    torch.cuda.synchronize()
    prepared = [t.clone() for t in ys]

    def step():
        outs, _, _ = bl.forward_grouped(mats, x, k, xq=xq, absmax=a)
        for t, o in zip(ys, outs):
            t.copy_(o)
        bl.quantize_acts(x16, xq16, a16)
        bl.forward(mats[0][0], mats[0][1], xq16, a16, 6912, k, y=y16)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in ys + [y16]]
    for o, e in zip(prepared, eager[:2]):
        check_equal(host(o).view(np.uint32), host(e).view(np.uint32), "grouped eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in ys + [y16]:
            t.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for t, e in zip(ys + [y16], eager):
            check_equal(host(t).view(np.uint32), host(e).view(np.uint32), f"grouped replay {rep}")


def test_two_streams_run_concurrently():
    # the library keeps no state between calls: two streams working at the same time on
    # different matrices give the results each gives alone
    print("case: two streams", flush=True)
    probs = []
    for i, (m, n, k) in enumerate(((1, 6912, 2560), (40, 1000, 2560))):
        w = synth.latent_weights(n, k, seed=9500 + i, device=DEV)
        packed, gamma = bl.quantize_weights(w)
        x = synth.activations(m, k, seed=9550 + i, dtype=torch.bfloat16, device=DEV)
        probs.append((packed, gamma, x, n, k))
    alone = []
    for packed, gamma, x, n, k in probs:
        (y, _, _) = bl.forward_fused(packed, gamma, x, n, k)
        torch.cuda.synchronize()
        alone.append(y.clone())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results = [[], []]
    for _ in range(8):
        for s, (packed, gamma, x, n, k), res in zip(streams, probs, results):
            with torch.cuda.stream(s):
                (y, _, _) = bl.forward_fused(packed, gamma, x, n, k)
                res.append(y)
    torch.cuda.synchronize()
    for res, ref in zip(results, alone):
        for y in res:
            check_equal(host(y).view(np.uint32), host(ref).view(np.uint32), "two streams")


def test_newer_entry_points_replay_in_a_graph():
    # the sub-layer normalisation (fused and two-kernel), the gated pair (fused and general
    # path with its workspace), the table-lookup and the binary decode, captured together
    print("case: graph replay of subln, gated pair, lut and binary calls", flush=True)
    k, n = 2560, 6912
    w = synth.latent_weights(n, k, seed=9500, device=DEV)
    packed, gamma = bl.quantize_weights(w)
    packed_b, beta = bl.quantize_weights_binary(w)
    w2 = synth.latent_weights(n, k, seed=9501, device=DEV)
    packed2, gamma2 = bl.quantize_weights(w2)
    del w, w2
    gain = synth.subln_gain(k, 9502, device=DEV)
    x1 = synth.activations(1, k, seed=9503, dtype=torch.bfloat16, device=DEV)
    x8 = synth.activations(8, k, seed=9504, dtype=torch.bfloat16, device=DEV)
    bufs = {}

    def buf(name, shape, dtype=torch.float32):
        if name not in bufs:
            bufs[name] = torch.empty(shape, dtype=dtype, device=DEV)
        return bufs[name]

    ws = torch.empty(bl.lib().bitlinear_gated_relu2_workspace_bytes(8, n), dtype=torch.uint8, device=DEV)
    outs = ["y_subln1", "y_subln8", "h1", "h8", "y_lut", "y_bin"]

    def step():
        xq1, a1 = buf("xq1", (1, bl.k_pad(k)), torch.int8), buf("a1", (1,))
        xq8, a8 = buf("xq8", (8, bl.k_pad(k)), torch.int8), buf("a8", (8,))
        bl.forward_subln(packed, gamma, x1, n, k, gain, 1e-5, y=buf("y_subln1", (1, n)), xq=xq1, scale=a1)
        bl.subln_quantize_acts(x8, gain, 1e-5, xq8, a8)
        bl.forward(packed, gamma, xq8, a8, n, k, y=buf("y_subln8", (8, n)))
        bl.forward_gated_relu2((packed, gamma), (packed2, gamma2), x1, n, k, subln=True, gain=gain, h=buf("h1", (1, n)),
                               xq=xq1, scale=a1)
        bl.forward_gated_relu2((packed, gamma), (packed2, gamma2), x8, n, k, h=buf("h8", (8, n)), xq=xq8, scale=a8,
                               workspace=ws)
        bl.quantize_acts(x1, xq1, a1)
        bl.forward_lut(packed, gamma, xq1, a1, n, k, y=buf("y_lut", (1, n)))
        bl.forward_binary(packed_b, beta, xq1, a1, n, k, y=buf("y_bin", (1, n)))

    step()
    torch.cuda.synchronize()
    eager = {o: bufs[o].clone() for o in outs}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for o in outs:
            bufs[o].fill_(float("nan"))
        scratch = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for o in outs:
            check_equal(host(bufs[o]).view(np.uint32), host(eager[o]).view(np.uint32), f"{o} replay {rep}")
