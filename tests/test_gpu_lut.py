"""GPU parity of the table-lookup decode kernel (bitlinear_forward_lut) against the oracle.

Same bars as bitlinear_forward: int32 accumulators bit-exact, y within 1e-5 relative."""
import numpy as np
import pytest
import torch

import bitlinear_fwd_amd as bl
import oracle
from bitlinear_fwd_amd import synth
from gpu_helpers import acts_host_f32, check_equal, check_y, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("m,n,k", [(1, 6912, 2560), (1, 2560, 6912), (1, 16, 256), (1, 17, 300), (2, 130, 1000),
                                   (3, 48, 2304), (4, 520, 2048), (1, 33, 8), (1, 1000, 8192), (2, 64, 3600),
                                   (4, 24, 512)])
def test_forward_lut(m, n, k):
    plan = bl.forward_lut_plan(m, n, k)
    print("case: lut", m, n, k, plan, flush=True)
    assert plan is not None
    rng = np.random.default_rng(m * 7 + n + k)
    q = rng.integers(-1, 2, (n, k)).astype(np.int8)
    packed = torch.from_numpy(oracle.pack(q)).to(DEV)
    x = synth.activations(m, k, seed=n + k, dtype=torch.bfloat16, device=DEV, outlier_p=0.01, outlier_mult=20.0)
    if m > 2:
        x[1] = 0
    xq, a = bl.quantize_acts(x)
    gamma = np.float32(0.0173)
    y, acc = bl.forward_lut(packed, torch.tensor([gamma], device=DEV), xq, a, n, k, want_y=True, want_acc=True)
    torch.cuda.synchronize()
    xq_ref, a_ref = oracle.quant_acts(acts_host_f32(x))
    check_equal(host(xq), xq_ref, "lut xq")
    acc_ref, y_ref = oracle.forward(q, gamma, xq_ref, a_ref, k)
    check_equal(host(acc), acc_ref, f"lut acc m={m} n={n} k={k}")
    check_y(host(y), y_ref, f"lut y m={m} n={n} k={k}")


def test_forward_lut_extreme_codes():
    # all +1 and all -1 rows against +-127 activations: the table entries reach +-254
    k, n = 2560, 32
    q = np.ones((n, k), np.int8)
    q[1::2] = -1
    packed = torch.from_numpy(oracle.pack(q)).to(DEV)
    xq = torch.full((1, bl.k_pad(k)), 127, dtype=torch.int8, device=DEV)
    xq[0, k:] = 0
    a = torch.ones(1, device=DEV)
    acc = bl.forward_lut(packed, torch.ones(1, device=DEV), xq, a, n, k, want_y=False, want_acc=True)
    torch.cuda.synchronize()
    assert np.all(host(acc)[0, 0::2] == 127 * k) and np.all(host(acc)[0, 1::2] == -127 * k)


def test_forward_lut_unsupported_shapes():
    assert bl.forward_lut_plan(5, 64, 256) is None          # more than four tokens
    assert bl.forward_lut_plan(4, 64, 28672) is None        # tables beyond the LDS budget
    packed = torch.zeros(bl.packed_bytes(64, 256), dtype=torch.uint8, device=DEV)
    xq = torch.zeros((5, 256), dtype=torch.int8, device=DEV)
    with pytest.raises(bl.BitLinearError):
        bl.forward_lut(packed, torch.ones(1, device=DEV), xq, torch.ones(5, device=DEV), 64, 256)
