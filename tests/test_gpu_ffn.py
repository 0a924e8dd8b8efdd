"""GPU parity of the gate / up pair with the squared-ReLU gating (feed-forward epilogue).

The aratech.ae article ("BitLinear: the building block") gives the feed-forward layers a
squared ReLU; for a gate / up pair of one input the library and the oracle read it as
h = relu(y_gate)^2 * y_up.  Bars: codes bit-exact (scale bit-exact, or within one fp32
ulp behind the sub-layer normalisation); h within 1e-5 relative of the oracle's fp64
value and exactly 0 where the gate is not positive.
"""
import numpy as np
import pytest
import torch

import bitlinear_fwd_amd as bl
import oracle
from bitlinear_fwd_amd import synth
from gpu_helpers import acts_host_f32, check_equal, check_y, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _announce(*a):
    print("case:", *a, flush=True)


def _ffn_check(m, n, k, dtype, subln, seed, unaligned=False):
    rng = np.random.default_rng(seed)
    qg, qu = (rng.integers(-1, 2, (n, k)).astype(np.int8) for _ in range(2))
    gg, gu = np.float32(0.0211), np.float32(0.0187)
    gate = (torch.from_numpy(oracle.pack(qg)).to(DEV), torch.tensor([gg], device=DEV))
    up = (torch.from_numpy(oracle.pack(qu)).to(DEV), torch.tensor([gu], device=DEV))
    if unaligned:
        flat = synth.activations(1, m * k + 1, seed=seed, dtype=dtype, device=DEV).reshape(-1)
        x = flat[1:].view(m, k)
    else:
        x = synth.activations(m, k, seed=seed, dtype=dtype, device=DEV, outlier_p=0.01, outlier_mult=20.0)
    if m > 2:
        x[1] = 0
    gain = None
    if subln:
        gain = torch.from_numpy(np.random.default_rng(seed + 1).uniform(0.5, 1.5, k).astype(np.float32)).to(DEV)
    h, xq, sc = bl.forward_gated_relu2(gate, up, x, n, k, subln=subln, gain=gain, eps=1e-5)
    torch.cuda.synchronize()
    if subln:
        xq_ref, sc_ref, _, _ = oracle.subln_quant_acts(acts_host_f32(x), host(gain), 1e-5)
        ulps = np.abs(host(sc).view(np.int32).astype(np.int64) - sc_ref.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1, f"scale {host(sc)} vs {sc_ref}"
    else:
        xq_ref, sc_ref = oracle.quant_acts(acts_host_f32(x))
        check_equal(host(sc).view(np.uint32), sc_ref.view(np.uint32), f"ffn absmax m={m} k={k}")
    check_equal(host(xq), xq_ref, f"ffn xq m={m} k={k}")
    h_ref = oracle.ffn_gate_up(qg, gg, qu, gu, xq_ref, sc_ref, k)
    check_y(host(h), h_ref, f"ffn h m={m} n={n} k={k}")
    assert np.count_nonzero(h_ref) > 0


@pytest.mark.parametrize("m,n,k,dtype,subln", [
    (1, 6912, 2560, torch.bfloat16, False),   # gate / up of a 2B-class layer
    (1, 6912, 2560, torch.bfloat16, True),
    (2, 700, 4096, torch.float32, False),
    (3, 300, 1000, torch.bfloat16, False),
    (3, 48, 1000, torch.float32, True),
    (4, 130, 2048, torch.bfloat16, True),
    (1, 33, 8, torch.bfloat16, False),
    (1, 28672, 8192, torch.bfloat16, False),  # 100B-class up projection
    # 257..512 row blocks, short runs: both weight runs issued as soon as the activations land
    (2, 6912, 2560, torch.bfloat16, False), (3, 6912, 2560, torch.float32, True),
    (4, 8192, 2048, torch.bfloat16, True), (2, 8192, 4096, torch.float32, False),
])
def test_gated_pair_one_kernel(m, n, k, dtype, subln):
    plan = bl.forward_gated_relu2_plan(m, n, k, "bf16" if dtype == torch.bfloat16 else "f32", subln)
    _announce("gated pair", m, n, k, dtype, subln, plan)
    assert plan["kernel"] == "fused"
    _ffn_check(m, n, k, dtype, subln, seed=m * 19 + n + k)


@pytest.mark.parametrize("m,n,k,dtype,subln,unaligned", [
    (8, 300, 2560, torch.bfloat16, False, False),   # more tokens: quantiser, two forwards, gating
    (16, 512, 2560, torch.bfloat16, True, False),
    (40, 130, 1000, torch.float32, False, False),   # 17..64 tokens: token groups
    (100, 130, 1000, torch.bfloat16, True, False),  # prefill sizes
    (1, 64, 300, torch.bfloat16, False, False),     # K not a multiple of 8
    (2, 64, 1024, torch.bfloat16, True, True),      # unaligned x
])
def test_gated_pair_general_path(m, n, k, dtype, subln, unaligned):
    plan = bl.forward_gated_relu2_plan(m, n, k, "bf16" if dtype == torch.bfloat16 else "f32", subln)
    _announce("gated pair general", m, n, k, dtype, subln, unaligned, plan)
    assert unaligned or plan["kernel"] != "fused"
    _ffn_check(m, n, k, dtype, subln, seed=m * 23 + n + k, unaligned=unaligned)


def test_gated_pair_needs_workspace_off_the_fused_path():
    k, n, m = 2560, 64, 8
    q = torch.zeros(bl.packed_bytes(n, k), dtype=torch.uint8, device=DEV)
    g = torch.ones(1, device=DEV)
    x = torch.ones((m, k), dtype=torch.bfloat16, device=DEV)
    h = torch.empty((m, n), device=DEV)
    xq = torch.empty((m, bl.k_pad(k)), dtype=torch.int8, device=DEV)
    sc = torch.empty(m, device=DEV)
    st = bl.lib().bitlinear_forward_gated_relu2(q.data_ptr(), g.data_ptr(), q.data_ptr(), g.data_ptr(), x.data_ptr(),
                                                bl.BL_BF16, m, n, k, 0, None, 0.0, h.data_ptr(), xq.data_ptr(),
                                                sc.data_ptr(), None, 0, None)
    assert st == bl.BL_ERR_INVALID_ARG
