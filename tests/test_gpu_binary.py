"""GPU parity of the 1-bit sign-binary variant (lpnh.cn section 2.1) against the oracle.

Bars: packed bytes, beta and int32 accumulators bit-exact; y within 1e-5 relative."""
import numpy as np
import pytest
import torch

import bitlinear_fwd_amd as bl
import oracle
from bitlinear_fwd_amd import synth
from gpu_helpers import acts_host_f32, check_equal, check_y, gamma_bits, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("n,k", [(1, 1), (16, 512), (17, 300), (33, 513), (100, 1000), (2560, 6912), (64, 2048)])
def test_binary_weight_quant(n, k):
    print("case: binary wq", n, k, flush=True)
    w = synth.latent_weights(n, k, seed=n + k)
    w[0, 0] = 0.0
    if k > 1:
        w[0, 1] = -0.0
    packed, beta = bl.quantize_weights_binary(w.to(DEV))
    torch.cuda.synchronize()
    beta_ref, _, packed_ref = oracle.quantize_weights_binary(w.numpy())
    assert gamma_bits(host(beta)) == gamma_bits(beta_ref)
    check_equal(host(packed), packed_ref, f"binary packed {n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1, 6912, 2560), (1, 2560, 6912), (2, 130, 1000), (3, 48, 300), (4, 520, 2048),
                                   (1, 33, 8), (1, 28672, 8192), (4, 64, 512), (2, 17, 4100)])
def test_forward_binary(m, n, k):
    plan = bl.forward_binary_plan(m, n, k)
    print("case: binary forward", m, n, k, plan, flush=True)
    assert plan is not None
    rng = np.random.default_rng(m * 5 + n + k)
    q = np.where(rng.random((n, k)) < 0.5, 1, -1).astype(np.int8)
    packed = torch.from_numpy(oracle.pack_binary(q)).to(DEV)
    x = synth.activations(m, k, seed=n + 2 * k, dtype=torch.bfloat16, device=DEV, outlier_p=0.01, outlier_mult=20.0)
    if m > 2:
        x[1] = 0
    xq, a = bl.quantize_acts(x)
    beta = np.float32(0.0159)
    y, acc = bl.forward_binary(packed, torch.tensor([beta], device=DEV), xq, a, n, k, want_y=True, want_acc=True)
    torch.cuda.synchronize()
    xq_ref, a_ref = oracle.quant_acts(acts_host_f32(x))
    check_equal(host(xq), xq_ref, "binary xq")
    acc_ref, y_ref = oracle.forward(q, beta, xq_ref, a_ref, k)
    check_equal(host(acc), acc_ref, f"binary acc m={m} n={n} k={k}")
    check_y(host(y), y_ref, f"binary y m={m} n={n} k={k}")


def test_binary_end_to_end_and_closed_form():
    n, k, m = 48, 1000, 2
    w = synth.latent_weights(n, k, seed=77)
    w[0] = torch.abs(w[0])  # row 0 all +1: acc = sum of the codes
    packed, beta = bl.quantize_weights_binary(w.to(DEV))
    x = synth.activations(m, k, seed=78, dtype=torch.float32, device=DEV)
    xq, a = bl.quantize_acts(x)
    y, acc = bl.forward_binary(packed, beta, xq, a, n, k, want_y=True, want_acc=True)
    torch.cuda.synchronize()
    beta_ref, q_ref, _ = oracle.quantize_weights_binary(w.numpy())
    xq_ref, a_ref = oracle.quant_acts(acts_host_f32(x))
    acc_ref, y_ref = oracle.forward(q_ref, beta_ref, xq_ref, a_ref, k)
    check_equal(host(acc), acc_ref, "binary e2e acc")
    check_y(host(y), y_ref, "binary e2e y")
    assert host(acc)[:, 0].tolist() == xq_ref[:, :k].astype(np.int64).sum(axis=1).tolist()


def test_binary_unsupported():
    assert bl.forward_binary_plan(5, 64, 512) is None
    packed = torch.zeros(bl.packed_bytes_binary(64, 512), dtype=torch.uint8, device=DEV)
    xq = torch.zeros((5, 512), dtype=torch.int8, device=DEV)
    with pytest.raises(bl.BitLinearError):
        bl.forward_binary(packed, torch.ones(1, device=DEV), xq, torch.ones(5, device=DEV), 64, 512)
