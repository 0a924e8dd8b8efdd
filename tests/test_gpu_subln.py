"""GPU parity of the sub-layer normalisation in front of the activation quantiser.

The aratech.ae article ("BitLinear: the building block") puts a simplified LayerNorm
right before activation quantisation; the library and the oracle read it as RMS
normalisation with a per-feature gain and eps.  Bars: codes and int32 accumulators
bit-exact; the scale within one fp32 ulp of the oracle's (both round an fp64 value once,
from sums of squares taken in different orders); y within 1e-5 relative.
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


def _gain(k, seed, kind):
    """'none', 'pos' (0.5..1.5), 'signed' (-2..2 with exact zeros), or 'unaligned' (a
    signed gain at a 4-byte offset, which takes the scalar and two-kernel paths)."""
    if kind == "none":
        return None, None
    rng = np.random.default_rng(seed)
    if kind == "pos":
        g = rng.uniform(0.5, 1.5, k).astype(np.float32)
    else:
        g = rng.uniform(-2.0, 2.0, k).astype(np.float32)
        g[rng.random(k) < 0.02] = 0.0
    if kind == "unaligned":
        buf = torch.empty(k + 1, dtype=torch.float32, device=DEV)
        buf[1:] = torch.from_numpy(g).to(DEV)
        return buf[1:], g
    return torch.from_numpy(g).to(DEV), g


def _acts(m, k, dtype, seed):
    x = synth.activations(m, k, seed=seed, dtype=dtype, device=DEV, outlier_p=0.01, outlier_mult=20.0)
    if m > 2:
        x[1] = 0  # a zero row: zero codes, zero scale
    return x


def check_scale(sc_gpu: np.ndarray, sc_ref: np.ndarray, what: str) -> None:
    a = sc_gpu.astype(np.float32).view(np.int32).astype(np.int64)
    b = sc_ref.astype(np.float32).view(np.int32).astype(np.int64)
    ulps = np.abs(a - b)
    assert np.all((sc_ref == 0) == (sc_gpu == 0)), f"{what}: zero pattern differs"
    assert ulps.max(initial=0) <= 1, f"{what}: {int(ulps.max())} ulps, {sc_gpu} vs {sc_ref}"


def _ref(x, g_host, eps):
    return oracle.subln_quant_acts(acts_host_f32(x), g_host, eps)


# ------------------------------------------------------------------ standalone quantiser
@pytest.mark.parametrize("m,k,dtype,gain", [
    (1, 2560, torch.bfloat16, "pos"), (1, 2560, torch.bfloat16, "none"), (3, 777, torch.float32, "signed"),
    (16, 6912, torch.bfloat16, "signed"), (5, 40000, torch.bfloat16, "pos"), (2, 8200, torch.float32, "signed"),
    (4, 8, torch.bfloat16, "signed"), (7, 1000, torch.bfloat16, "unaligned"), (64, 2560, torch.bfloat16, "pos"),
    (2, 32776, torch.float32, "none"),
])
@pytest.mark.parametrize("eps", [1e-5, 0.0])
def test_subln_quantize_acts(m, k, dtype, gain, eps):
    _announce("subln quant", m, k, dtype, gain, eps)
    x = _acts(m, k, dtype, seed=m * 7 + k)
    g_dev, g_host = _gain(k, seed=k, kind=gain)
    xq, sc = bl.subln_quantize_acts(x, g_dev, eps)
    torch.cuda.synchronize()
    xq_ref, sc_ref, _, _ = _ref(x, g_host, eps)
    check_equal(host(xq), xq_ref, f"subln xq m={m} k={k}")
    check_scale(host(sc), sc_ref, f"subln scale m={m} k={k}")


def test_subln_quantize_closed_forms():
    # a constant row normalises to +-1 everywhere: codes +-127 and scale 1; one non-zero
    # feature v normalises to sqrt(K): scale sqrt(K) (eps = 0)
    k = 4096
    x = torch.zeros((3, k), dtype=torch.float32, device=DEV)
    x[0] = 0.75
    x[1] = -3.0
    x[2, 100] = -2.5
    xq, sc = bl.subln_quantize_acts(x, None, 0.0)
    torch.cuda.synchronize()
    xq, sc = host(xq), host(sc)
    assert np.all(xq[0, :k] == 127) and np.all(xq[1, :k] == -127)
    assert sc[0] == 1.0 and sc[1] == 1.0
    assert xq[2, 100] == -127 and np.count_nonzero(xq[2]) == 1 and sc[2] == np.float32(64.0)


def test_subln_matches_plain_quantiser_without_gain():
    # no gain: the codes are those of the plain quantiser, bit for bit
    x = _acts(6, 2560, torch.bfloat16, seed=5)
    xq0, a0 = bl.quantize_acts(x)
    xq1, sc = bl.subln_quantize_acts(x, None, 1e-5)
    torch.cuda.synchronize()
    check_equal(host(xq1), host(xq0), "subln vs plain codes")
    assert np.all(host(sc)[host(a0) == 0] == 0)


def test_subln_argument_errors():
    x = torch.ones((2, 256), dtype=torch.float32, device=DEV)
    with pytest.raises(bl.BitLinearError):
        bl.subln_quantize_acts(x, None, -1.0)
    with pytest.raises(bl.BitLinearError):
        bl.subln_quantize_acts(x, None, float("nan"))
    with pytest.raises(ValueError):
        bl.subln_quantize_acts(x, torch.ones(255, dtype=torch.float32, device=DEV), 1e-5)


# ------------------------------------------------------------------ normalise + quantise + forward
def _subln_fwd_check(m, n, k, dtype, gain, eps, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, (n, k)).astype(np.int8)
    packed = torch.from_numpy(oracle.pack(q)).to(DEV)
    x = _acts(m, k, dtype, seed)
    g_dev, g_host = _gain(k, seed + 1, gain)
    gamma = np.float32(0.0159577)
    (y, acc), xq, sc = bl.forward_subln(packed, torch.tensor([gamma], device=DEV), x, n, k, g_dev, eps,
                                        want_y=True, want_acc=True)
    torch.cuda.synchronize()
    xq_ref, sc_ref, _, _ = _ref(x, g_host, eps)
    check_equal(host(xq), xq_ref, f"subln fwd xq m={m} k={k}")
    check_scale(host(sc), sc_ref, f"subln fwd scale m={m} k={k}")
    acc_ref, y_ref = oracle.forward(q, gamma, xq_ref, sc_ref, k)
    check_equal(host(acc), acc_ref, f"subln fwd acc m={m} n={n} k={k}")
    check_y(host(y), y_ref, f"subln fwd y m={m} n={n} k={k}")


@pytest.mark.parametrize("m,n,k,dtype", [
    (1, 6912, 2560, torch.bfloat16), (1, 2560, 6912, torch.bfloat16), (1, 700, 28672, torch.bfloat16),
    (2, 130, 4096, torch.bfloat16), (3, 48, 1000, torch.float32), (4, 520, 2048, torch.bfloat16),
    (1, 33, 8, torch.bfloat16), (2, 100, 1000, torch.float32), (4, 24, 1024, torch.float32),
    (3, 300, 2304, torch.bfloat16),
    # 257..512 row blocks with short runs: weights issued as soon as the activations land
    (2, 6912, 2560, torch.bfloat16), (4, 8192, 2048, torch.float32), (3, 4100, 1000, torch.bfloat16),
])
@pytest.mark.parametrize("gain", ["signed", "none"])
def test_forward_subln_single_kernel(m, n, k, dtype, gain):
    plan = bl.forward_subln_plan(m, n, k, "bf16" if dtype == torch.bfloat16 else "f32")
    _announce("forward subln", m, n, k, dtype, gain, plan)
    assert plan["kernel"] == "fused" and plan["acts"] == "registers"
    _subln_fwd_check(m, n, k, dtype, gain, 1e-5, seed=m * 31 + n + k)


@pytest.mark.parametrize("m,n,k,dtype,gain", [
    (5, 64, 512, torch.bfloat16, "signed"), (16, 300, 2560, torch.bfloat16, "pos"),
    (1, 64, 300, torch.bfloat16, "signed"), (4, 30, 20000, torch.bfloat16, "pos"),
    (3, 40, 12000, torch.float32, "none"), (2, 64, 1000, torch.bfloat16, "unaligned"),
    (40, 72, 700, torch.float32, "signed"), (100, 72, 700, torch.bfloat16, "pos"),
])
def test_forward_subln_two_kernels(m, n, k, dtype, gain):
    # outside the one-kernel path: the normalising quantiser, then the forward kernel
    plan = bl.forward_subln_plan(m, n, k, "bf16" if dtype == torch.bfloat16 else "f32")
    _announce("forward subln two kernels", m, n, k, dtype, gain, plan)
    assert gain == "unaligned" or plan["kernel"] != "fused"
    _subln_fwd_check(m, n, k, dtype, gain, 1e-5, seed=m * 13 + n + k)


@pytest.mark.parametrize("m,ns,k,dtype", [
    (1, [2560, 640, 640], 2560, torch.bfloat16),       # Q, K, V behind one normalisation
    (1, [6912, 6912], 2560, torch.bfloat16),           # gate + up
    (3, [17, 300, 1000], 1000, torch.float32),
    (8, [300, 100], 2560, torch.bfloat16),             # more tokens: two-kernel path
    (2, [2560, 2560], 2560, torch.bfloat16),           # 320 row blocks: weights issued as activations land
    (1, [6912], 2560, torch.bfloat16),                 # a group of one, 432 row blocks
])
def test_forward_grouped_subln(m, ns, k, dtype):
    _announce("forward grouped subln", m, ns, k, dtype)
    rng = np.random.default_rng(m + k)
    qs = [rng.integers(-1, 2, (n, k)).astype(np.int8) for n in ns]
    gammas = [np.float32(0.01 + 0.001 * i) for i in range(len(ns))]
    x = _acts(m, k, dtype, seed=k + 3)
    g_dev, g_host = _gain(k, seed=k + 4, kind="signed")
    mats = [(torch.from_numpy(oracle.pack(q)).to(DEV), torch.tensor([g], device=DEV), n)
            for q, g, n in zip(qs, gammas, ns)]
    outs, xq, sc = bl.forward_grouped_subln(mats, x, k, g_dev, 1e-5, want_y=True, want_acc=True)
    torch.cuda.synchronize()
    xq_ref, sc_ref, _, _ = _ref(x, g_host, 1e-5)
    check_equal(host(xq), xq_ref, f"grouped subln xq m={m} k={k}")
    check_scale(host(sc), sc_ref, f"grouped subln scale m={m} k={k}")
    for i, ((y, acc), q, g) in enumerate(zip(outs, qs, gammas)):
        acc_ref, y_ref = oracle.forward(q, g, xq_ref, sc_ref, k)
        check_equal(host(acc), acc_ref, f"grouped subln acc {i}")
        check_y(host(y), y_ref, f"grouped subln y {i}")
