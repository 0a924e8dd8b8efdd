"""End-to-end parity at the workloads' full sizes, in the launch configuration the
benchmark times (the same C ABI calls, M decides decode or prefill kernel).

Weights and activations are drawn on the GPU with the seeded generators, the whole path
runs on the GPU (weight quantiser, activation quantiser, forward), and the oracle runs on
host copies of the same inputs.  Every stage is compared bit-exactly (gamma, packed
bytes, xq, absmax, int32 acc) and y within 1e-5 relative, on every output: the oracle's
contraction runs on host threads over slices of the token rows where M is large (the
2048-token prefill)."""
import numpy as np
import pytest
import torch

import bitlinear_fwd_amd as bl
import oracle
from bitlinear_fwd_amd import synth
from gpu_helpers import acts_host_f32, check_equal, check_y, gamma_bits, host, oracle_forward_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(workload: int, layer: int, midx: int, k: int, n: int, m: int):
    wl = synth.WORKLOADS[workload]
    print(f"case: workload {workload} layer {layer} matrix {midx} K={k} N={n} M={m}", flush=True)
    w_dev = synth.latent_weights(n, k, seed=synth.weight_seed(workload, layer, midx), device=DEV)
    x_dev = synth.activations(m, k, seed=synth.act_seed(workload, layer, midx), dtype=wl.act_dtype, device=DEV,
                              outlier_p=wl.outlier_p, outlier_mult=wl.outlier_mult)
    packed, gamma = bl.quantize_weights(w_dev)
    xq, a = bl.quantize_acts(x_dev)
    y, acc = bl.forward(packed, gamma, xq, a, n, k, want_y=True, want_acc=True)
    torch.cuda.synchronize()
    w = host(w_dev)
    del w_dev
    g_ref = oracle.gamma_absmean(w)
    assert gamma_bits(host(gamma)) == gamma_bits(g_ref)
    q_ref = oracle.ternarise(w, g_ref)
    del w
    check_equal(host(packed), oracle.pack(q_ref), "packed")
    xq_ref, a_ref = oracle.quant_acts(acts_host_f32(x_dev))
    xq_h, a_h, acc_h, y_h = host(xq), host(a), host(acc), host(y)
    check_equal(xq_h, xq_ref, "xq")
    check_equal(a_h.view(np.uint32), a_ref.view(np.uint32), "absmax")
    acc_ref, y_ref = oracle_forward_rows(q_ref, g_ref, xq_ref, a_ref, k)
    check_equal(acc_h, acc_ref, "acc")
    check_y(y_h, y_ref)


def _run_fused(workload: int, layer: int, midx: int, k: int, n: int, m: int):
    # the one-call quantise + forward path on the same inputs as _run
    wl = synth.WORKLOADS[workload]
    print(f"case: fused workload {workload} layer {layer} matrix {midx} K={k} N={n} M={m}", flush=True)
    w_dev = synth.latent_weights(n, k, seed=synth.weight_seed(workload, layer, midx), device=DEV)
    x_dev = synth.activations(m, k, seed=synth.act_seed(workload, layer, midx), dtype=wl.act_dtype, device=DEV,
                              outlier_p=wl.outlier_p, outlier_mult=wl.outlier_mult)
    packed, gamma = bl.quantize_weights(w_dev)
    (y, acc), xq, a = bl.forward_fused(packed, gamma, x_dev, n, k, want_y=True, want_acc=True)
    torch.cuda.synchronize()
    w = host(w_dev)
    del w_dev
    g_ref = oracle.gamma_absmean(w)
    q_ref = oracle.ternarise(w, g_ref)
    del w
    xq_ref, a_ref = oracle.quant_acts(acts_host_f32(x_dev))
    check_equal(host(xq), xq_ref, "fused xq")
    check_equal(host(a).view(np.uint32), a_ref.view(np.uint32), "fused absmax")
    acc_ref, y_ref = oracle.forward(q_ref, g_ref, xq_ref, a_ref, k)
    check_equal(host(acc), acc_ref, "fused acc")
    check_y(host(y), y_ref)


@pytest.mark.parametrize("midx", [0, 2])
def test_workload1_fused_m1(midx):
    _, k, n = synth.WORKLOADS[1].matrices[midx]
    _run_fused(1, 0, midx, k, n, 1)


def test_workload0_single_bitlinear():
    _run(0, 0, 0, 256, 512, 1)


@pytest.mark.parametrize("midx", [0, 1, 2])
def test_workload1_2b_decode_m1(midx):
    _, k, n = synth.WORKLOADS[1].matrices[midx]
    _run(1, 0, midx, k, n, 1)


@pytest.mark.parametrize("midx", range(7))
def test_workload2_2b_layer_m16(midx):
    _, k, n = synth.WORKLOADS[2].matrices[midx]
    _run(2, 0, midx, k, n, 16)


@pytest.mark.parametrize("midx", [0, 1])
def test_workload3_prefill_m2048(midx):
    # all 2048 x N outputs: the up projection runs one K group per 64 x 192 tile, the down
    # projection two K groups that exchange their int32 partials through LDS
    _, k, n = synth.WORKLOADS[3].matrices[midx]
    _run(3, 0, midx, k, n, 2048)


@pytest.mark.parametrize("m", [1, 8])
@pytest.mark.parametrize("midx", [0, 1])
def test_workload4_100b_decode(midx, m):
    _, k, n = synth.WORKLOADS[4].matrices[midx]
    _run(4, 0, midx, k, n, m)


@pytest.mark.parametrize("midx", [0, 1])
def test_workload4_fused_m1(midx):
    # the benchmark's call for one token on the 100B-class shapes: one fused launch
    _, k, n = synth.WORKLOADS[4].matrices[midx]
    assert bl.forward_fused_plan(1, n, k, "bf16")["kernel"] == "fused"
    _run_fused(4, 0, midx, k, n, 1)


@pytest.mark.parametrize("m", [1, 8])
@pytest.mark.parametrize("midx", [0, 1])
def test_workload5_one_of_8_shard(midx, m):
    # one GPU's shard of the 100B-class matrices: 3584 output rows of the up projection,
    # 3584 input columns of the down projection (whose partial sums an all-reduce would add)
    _, k, n = synth.WORKLOADS[5].matrices[midx]
    _run(5, 0, midx, k, n, m)
    if m == 1:
        _run_fused(5, 0, midx, k, n, 1)
