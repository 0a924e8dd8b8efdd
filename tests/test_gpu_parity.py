"""GPU parity of every step against the CPU oracle, through the C ABI (ctypes binding).

Stage-wise: each kernel is fed bytes the oracle also consumes (device tensors copied to
the host), so a mismatch names the stage.  End-to-end cases live in test_gpu_workloads.py.
"""
import json
import os

import numpy as np
import pytest
import torch

import bitlinear_fwd_amd as bl
import oracle
from bitlinear_fwd_amd import synth
from gpu_helpers import acts_host_f32, check_equal, check_y, gamma_bits, host, oracle_forward_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _announce(*a):
    print("case:", *a, flush=True)


# ------------------------------------------------------------------ weight quantiser
def _wq_check(w_dev: torch.Tensor, tag: str):
    packed, gamma = bl.quantize_weights(w_dev)
    torch.cuda.synchronize()
    w = host(w_dev)
    g_ref, q_ref, p_ref = oracle.quantize_weights(w)
    assert gamma_bits(host(gamma)) == gamma_bits(g_ref), (tag, float(host(gamma)[0]), float(g_ref))
    check_equal(host(packed), p_ref, f"packed {tag}")
    return packed, gamma, q_ref, g_ref


@pytest.mark.parametrize("n,k", [(1, 1), (16, 256), (17, 300), (33, 513), (512, 256), (100, 1000),
                                 (64, 4103), (3, 70000), (1000, 3)])
def test_weight_quant_random(n, k):
    _announce("weight_quant", n, k)
    _wq_check(synth.latent_weights(n, k, seed=n * 7 + k, device=DEV), f"{n}x{k}")


def test_weight_quant_golden_ties():
    with open(os.path.join(GOLDEN, "quant_examples.json")) as f:
        cases = json.load(f)["weights"]
    for c in cases:
        _announce("weight_quant golden", c["W"])
        w = torch.tensor(c["W"], dtype=torch.float32, device=DEV)
        packed, gamma, q_ref, _ = _wq_check(w, str(c["W"]))
        assert float(host(gamma)[0]) == c["gamma"]
        n, k = w.shape
        assert oracle.unpack(host(packed), n, k).tolist() == c["q"]


def test_weight_quant_wide_range_and_subnormals():
    rng = np.random.default_rng(5)
    for trial in range(6):
        _announce("weight_quant wide", trial)
        n, k = int(rng.integers(1, 40)), int(rng.integers(1, 700))
        w = (rng.standard_normal((n, k)) * 10.0 ** rng.uniform(-44, 37, (n, k))).astype(np.float32)
        if trial == 3:
            w[:] = np.float32(1e-45) * rng.integers(0, 5, (n, k))  # subnormal-only tensor
        _wq_check(torch.from_numpy(w).to(DEV), f"wide{trial}")


def test_weight_quant_special_tensors():
    for name, w in [("zeros", np.zeros((16, 256), np.float32)),
                    ("const", np.full((20, 300), -0.03125, np.float32)),
                    ("one_hot", np.eye(17, 260, dtype=np.float32))]:
        _announce("weight_quant", name)
        _wq_check(torch.from_numpy(w).to(DEV), name)


def test_weight_quant_gamma_at_two_to_the_32_elements():
    # N * K = 2^32 elements (256 x 2^24), beyond the one-limb-at-a-time division: ones with
    # the first j entries set to 2 have the exact mean 1 + j * 2^-32.  One fp32 ulp at 1 is
    # 2^-23 = 2^9 * 2^-32, so j = 256 is exactly half an ulp (ties to the even 1.0), j = 257
    # is just above it (1 + 2^-23), and j = 768 is one and a half ulps (ties to the even
    # 1 + 2^-22).  The codes are not checked: gamma is the point.
    n, k = 256, 1 << 24
    w = torch.ones((n, k), dtype=torch.float32, device=DEV)
    for j, want in ((256, 0x3F800000), (257, 0x3F800001), (768, 0x3F800002)):
        _announce("weight_quant 2^32 elements", j)
        w.view(-1)[:j] = 2.0
        _, gamma = bl.quantize_weights(w)
        torch.cuda.synchronize()
        assert gamma_bits(host(gamma)) == want, (j, hex(gamma_bits(host(gamma))))
        w.view(-1)[:j] = 1.0
    del w
    torch.cuda.empty_cache()


def test_weight_quant_unaligned_source():
    _announce("weight_quant unaligned")
    base = synth.latent_weights(1, 33 * 256 + 1, seed=3, device=DEV).reshape(-1)
    w = base[1:].view(33, 256)  # 4-byte aligned, not 16-byte aligned: scalar load path
    assert w.data_ptr() % 16 != 0
    _wq_check(w, "unaligned")


def test_weight_quant_deterministic():
    w = synth.latent_weights(700, 2560, seed=99, device=DEV)
    p1, g1 = bl.quantize_weights(w)
    p2, g2 = bl.quantize_weights(w)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(g1, g2)


# ------------------------------------------------------------------ activation quantiser
def _aq_check(x_dev: torch.Tensor, tag: str):
    xq, a, rs = bl.quantize_acts(x_dev, want_rowsum=True)
    torch.cuda.synchronize()
    xq_ref, a_ref = oracle.quant_acts(acts_host_f32(x_dev))
    check_equal(host(a).view(np.uint32), a_ref.view(np.uint32), f"absmax {tag}")
    check_equal(host(xq), xq_ref, f"xq {tag}")
    # the optional row sums: exact sums of the oracle's codes
    check_equal(host(rs), xq_ref.astype(np.int64).sum(axis=1).astype(np.int32), f"rowsum {tag}")
    return xq, a, xq_ref, a_ref


@pytest.mark.parametrize("m,k,dtype", [(1, 256, torch.float32), (3, 300, torch.float32), (5, 2560, torch.bfloat16),
                                       (16, 6912, torch.bfloat16), (7, 1000, torch.bfloat16),
                                       (4, 999, torch.bfloat16), (2, 28672, torch.bfloat16),
                                       (9, 12000, torch.float32), (300, 64, torch.bfloat16),
                                       # 256 / 1024 threads per row, registers exactly full, re-read tail
                                       (1, 8192, torch.bfloat16), (2, 8200, torch.float32), (1, 32768, torch.bfloat16),
                                       (3, 32776, torch.bfloat16), (2, 40000, torch.float32)])
def test_act_quant(m, k, dtype):
    _announce("act_quant", m, k, dtype)
    x = synth.activations(m, k, seed=m * 131 + k, dtype=dtype, device=DEV, outlier_p=0.01, outlier_mult=20.0)
    _aq_check(x, f"{m}x{k}")


def test_act_quant_golden_and_zero_rows():
    with open(os.path.join(GOLDEN, "quant_examples.json")) as f:
        cases = json.load(f)["acts"]
    for c in cases:
        _announce("act_quant golden", c["x"])
        x = torch.tensor([c["x"]], dtype=torch.float32, device=DEV)
        xq, a, _, _ = _aq_check(x, str(c["x"]))
        assert host(xq)[0, : len(c["x"])].tolist() == c["xq"]
    x = synth.activations(6, 512, seed=1, dtype=torch.bfloat16, device=DEV)
    x[2] = 0
    _aq_check(x, "zero row")


def test_act_quant_unaligned_source():
    for dtype in (torch.float32, torch.bfloat16):
        _announce("act_quant unaligned", dtype)
        flat = synth.activations(1, 4 * 512 + 1, seed=4, dtype=dtype, device=DEV).reshape(-1)
        x = flat[1:].view(4, 512)
        assert x.data_ptr() % 16 != 0
        _aq_check(x, f"unaligned {dtype}")


def test_act_quant_every_bf16_value():
    # one token holding every finite bf16 value, plus rows scaled so the maximum varies
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f32(bits)
    keep = bits[np.isfinite(vals)]
    keep = keep[: len(keep) // 8 * 8]
    row = torch.from_numpy(keep.view(np.int16)).to(DEV).view(torch.bfloat16)
    small = row[(row.float().abs() <= 3.0)]
    small = small[: small.numel() // 8 * 8]
    for tag, x in [("all", row[None, :]), ("le3", small[None, :])]:
        _announce("act_quant bf16 sweep", tag)
        _aq_check(x.contiguous(), tag)


def _tie_rows(k):
    """Three activation rows whose products x * fl32(127 / a) land exactly on halves: row 0
    has max 127 (scale 1.0) and holds +-(n + 0.5) for n = 0..126; row 1 has max 63.5
    (scale 2.0) and holds +-(n / 2 + 0.25); row 2 is row 0 negated.  Every value is exact
    in bf16.  The expected
    codes are the round-half-to-even neighbours, written out here from the definition."""
    halves = np.arange(127, dtype=np.float64) + 0.5
    r0 = np.concatenate([[127.0], halves, -halves])
    r1 = np.concatenate([[63.5], halves / 2, -halves / 2])
    x = np.zeros((3, k), dtype=np.float32)
    x[0, : r0.size] = r0
    x[1, : r1.size] = r1
    x[2, : r0.size] = -r0
    even = lambda v: np.where(np.floor(v) % 2 == 0, np.floor(v), np.floor(v) + 1)  # v = n + 0.5 >= 0
    c = np.concatenate([[127], even(halves), -even(halves)]).astype(np.int8)
    want = np.zeros((3, k), dtype=np.int8)
    want[0, : c.size] = c
    want[1, : c.size] = c  # 2 * (n / 2 + 0.25) = n + 0.5: the same codes
    want[2, : c.size] = -c
    return x, want


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_act_quant_rounding_ties(dtype):
    # the quantisers round half to even: a product exactly on a half goes to the even code
    k = 256
    x_np, want = _tie_rows(k)
    x = torch.from_numpy(x_np).to(DEV).to(dtype)
    assert np.array_equal(acts_host_f32(x), x_np)  # exact in bf16
    _announce("act_quant ties", dtype)
    xq, a, xq_ref, _ = _aq_check(x, f"ties {dtype}")
    check_equal(xq_ref[:, :k], want, "oracle tie codes")
    check_equal(host(xq)[:, :k], want, "tie codes")
    # the fused forms quantise in the forward kernel: registers (one and 432 row blocks,
    # the second issuing its weights as soon as the activations land) and the LDS form
    for n, kk in ((512, k), (6912, k), (65600, 768)):
        xx = torch.zeros((3, kk), dtype=dtype, device=DEV)
        xx[:, :k] = x
        ww = np.zeros((3, kk), dtype=np.int8)
        ww[:, :k] = want
        q = np.random.default_rng(n).integers(-1, 2, (n, kk)).astype(np.int8)
        packed = torch.from_numpy(oracle.pack(q)).to(DEV)
        plan = bl.forward_fused_plan(3, n, kk, "bf16" if dtype == torch.bfloat16 else "f32")
        _announce("forward fused ties", n, kk, dtype, plan)
        assert plan["kernel"] == "fused"
        (y, acc), xq2, a2 = bl.forward_fused(packed, torch.tensor([0.02], device=DEV), xx, n, kk, want_y=True,
                                             want_acc=True)
        torch.cuda.synchronize()
        check_equal(host(xq2)[:, :kk], ww, f"fused tie codes n={n}")
        acc_ref, y_ref = oracle.forward(q, np.float32(0.02), host(xq2), host(a2), kk)
        check_equal(host(acc), acc_ref, f"fused tie acc n={n}")
        check_y(host(y), y_ref, f"fused tie y n={n}")
    # the sub-layer normalisation with no gain decides the codes on x itself: the same ties
    _announce("subln ties", dtype)
    xq3, _ = bl.subln_quantize_acts(x, None, 1e-5)
    (y3, acc3), xq4, _ = bl.forward_subln(packed, torch.tensor([0.02], device=DEV), xx, n, kk, None, 1e-5,
                                          want_y=True, want_acc=True)
    torch.cuda.synchronize()
    check_equal(host(xq3)[:, :k], want, "subln tie codes")
    check_equal(host(xq4)[:, :kk], ww, "fused subln tie codes")


def test_act_quant_deterministic():
    x = synth.activations(64, 6912, seed=8, dtype=torch.bfloat16, device=DEV, outlier_p=0.005, outlier_mult=30.0)
    a1 = bl.quantize_acts(x)
    a2 = bl.quantize_acts(x)
    torch.cuda.synchronize()
    assert torch.equal(a1[0], a2[0]) and torch.equal(a1[1], a2[1])


# ------------------------------------------------------------------ forward (contraction + rescale)
def _fwd_check(m, n, k, seed, want=("y", "acc")):
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, (n, k)).astype(np.int8)
    packed = oracle.pack(q)
    x = synth.activations(m, k, seed=seed, dtype=torch.float32, outlier_p=0.01, outlier_mult=20.0).numpy()
    if m > 2:
        x[m // 2] = 0  # a zero token
    xq, a = oracle.quant_acts(x)
    gamma = np.float32(0.0159577)
    acc_ref, y_ref = oracle.forward(q, gamma, xq, a, k)
    d = lambda arr: torch.from_numpy(arr).to(DEV)
    y, acc = bl.forward(d(packed), d(np.array([gamma], np.float32)), d(xq), d(a), n, k,
                        want_y=True, want_acc=True)
    torch.cuda.synchronize()
    check_equal(host(acc), acc_ref, f"acc m={m} n={n} k={k}")
    check_y(host(y), y_ref, f"y m={m} n={n} k={k}")


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 15, 16])
@pytest.mark.parametrize("n,k", [(16, 256), (17, 300), (512, 256), (130, 1000), (48, 2304), (1, 1)])
def test_forward_decode(m, n, k):
    _announce("forward decode", m, n, k)
    _fwd_check(m, n, k, seed=m * 1000 + n + k)


@pytest.mark.parametrize("m,n,k,acts,rb,run", [
    # M <= 4: activations in registers (DPP broadcast), every supported run length, exact
    # and ragged wave tilings, one to four tokens
    (1, 512, 256, "registers", 1, 1), (1, 16400, 300, "registers", 1, 2), (3, 130, 7000, "registers", 1, 2),
    (1, 64, 10000, "registers", 1, 3), (2, 8200, 12000, "registers", 1, 4), (4, 100, 16000, "registers", 1, 4),
    (1, 40, 17000, "registers", 1, 5), (2, 30, 22000, "registers", 1, 6), (1, 100, 27000, "registers", 1, 7),
    (2, 50, 30000, "registers", 1, 8), (1, 300, 40000, "registers", 1, 10), (3, 33, 47000, "registers", 1, 12),
    (1, 20, 55000, "registers", 1, 14), (4, 20, 62000, "registers", 1, 16), (2, 70, 5000, "registers", 1, 2),
    (3, 1000, 2560, "registers", 1, 2),
    # K beyond 16 waves x 16 tiles: activations loaded with each tile
    (4, 40, 70000, "per-tile loads", 1, 0),
    # M = 5..16 on rows over 4096: activations loaded with each tile, 1/2/4 row blocks
    (8, 2560, 6912, "per-tile loads", 1, 0), (7, 9000, 4100, "per-tile loads", 2, 0),
    (16, 4200, 9000, "per-tile loads", 1, 0), (6, 20000, 5000, "per-tile loads", 4, 0),
    # M = 5..16 on rows up to 4096: two-tile register runs (token group of 8 for M <= 8,
    # 16 above), 1 or 2 row blocks per workgroup
    (16, 16400, 256, "registers", 2, 2), (12, 16400, 1000, "registers", 2, 2), (9, 300, 512, "registers", 1, 2),
    (13, 7000, 4096, "registers", 2, 2), (16, 100, 3000, "registers", 1, 2), (11, 6150, 2560, "registers", 2, 2),
    (5, 8200, 300, "registers", 2, 2), (6, 20000, 1000, "registers", 2, 2), (8, 6912, 2560, "registers", 2, 2),
    (7, 100, 700, "registers", 1, 2), (8, 33, 4096, "registers", 1, 2)])
def test_forward_decode_variants(m, n, k, acts, rb, run):
    # every decode-kernel variant against the oracle, including ragged N and K
    plan = bl.forward_plan(m, n, k)
    _announce("forward decode variant", m, n, k, plan)
    assert plan["kernel"] == "decode" and plan["acts"] == acts and plan["row_blocks"] == rb
    assert plan["tiles_per_wave"] == run
    _fwd_check(m, n, k, seed=m * 7 + n * 3 + k)


@pytest.mark.parametrize("m", [17, 24, 32, 33, 48, 49, 64])
@pytest.mark.parametrize("n,k", [(16, 256), (17, 300), (130, 1000), (2560, 2560), (300, 6912), (1, 1), (6190, 700),
                                 (17000, 300)])
def test_forward_token_groups(m, n, k):
    # 17..64 tokens: the decode kernel with 2..4 token groups of 16 (the last one ragged)
    # sharing each decoded weight fragment, 1..8 waves, 1, 2 (6190 columns: 387 row blocks,
    # the last workgroup one short) or 4 row blocks per workgroup (17000: 1063 row blocks),
    # against the oracle on every output
    plan = bl.forward_plan(m, n, k)
    _announce("forward token groups", m, n, k, plan)
    assert plan["kernel"] == "decode" and plan["acts"] == "per-tile loads" and plan["threads"] <= 512
    _fwd_check(m, n, k, seed=m * 1000 + n + k)


@pytest.mark.parametrize("m,n,k,waves,rb", [(64, 6190, 4096, 4, 2), (17, 17000, 2048, 4, 4), (40, 17000, 2048, 2, 4),
                                            (33, 2560, 6912, 8, 1)])
def test_forward_token_groups_waves(m, n, k, waves, rb):
    # token groups with several waves per workgroup splitting K, and shared row blocks
    plan = bl.forward_plan(m, n, k)
    _announce("forward token groups waves", m, n, k, plan)
    assert plan["kernel"] == "decode" and plan["threads"] == 64 * waves and plan["row_blocks"] == rb
    _fwd_check(m, n, k, seed=m * 1000 + n + k)


@pytest.mark.parametrize("m,n,k", [(48, 30000, 512), (64, 24000, 1024)])
def test_forward_prefill_few_tokens(m, n, k):
    # 17..64 tokens where the token rows would be re-read by too many row blocks: the
    # prefill kernel (one 64-row tile high, two K groups), against the oracle on every output
    plan = bl.forward_plan(m, n, k)
    _announce("forward prefill few tokens", m, n, k, plan)
    assert plan["kernel"] == "prefill" and plan["k_groups"] == 2
    _fwd_check(m, n, k, seed=m * 1000 + n + k)


@pytest.mark.parametrize("m", [65, 100, 128, 129, 257])
@pytest.mark.parametrize("n,k", [(16, 256), (17, 300), (130, 1000), (300, 2304), (1, 1), (129, 513)])
def test_forward_prefill(m, n, k):
    _announce("forward prefill", m, n, k)
    _fwd_check(m, n, k, seed=m * 1000 + n + k)


@pytest.mark.parametrize("m,n,k,tile_n,k_groups", [
    (2048, 4100, 1000, 192, 1), (333, 24000, 2600, 192, 1), (2000, 4090, 1000, 256, 1), (3000, 9000, 700, 384, 1),
    (4096, 2560, 6912, 384, 1), (1792, 6912, 2560, 384, 1), (4000, 8190, 1000, 384, 1), (4096, 8192, 200, 384, 1),
    (2048, 2560, 6912, 192, 2),
    (1500, 2000, 777, 192, 2),
    # two K groups per tile where the tiles do not fill the chip; odd chunk counts (K = 1100:
    # 5 chunks, 6912: 27) leave the second group one chunk short
    (1000, 3000, 777, 192, 2), (700, 2600, 1100, 192, 2), (500, 7000, 1100, 256, 2), (450, 8000, 6912, 256, 2)])
def test_forward_prefill_tile_shapes(m, n, k, tile_n, k_groups):
    # the prefill tile shapes (64 x 256, 64 x 192 or the eight-wave 64 x 384 by the last
    # round's load, one or two K groups per tile) with ragged M, N and K; every output is
    # checked (the oracle's rows split over host threads)
    plan = bl.forward_plan(m, n, k)
    _announce("forward prefill tiles", m, n, k, plan)
    assert plan["kernel"] == "prefill" and plan["tile_m"] == 64 and plan["tile_n"] == tile_n
    assert plan["k_groups"] == k_groups and plan["threads"] == (512 if tile_n == 384 else 256 * k_groups)
    rng = np.random.default_rng(m + n + k)
    q = rng.integers(-1, 2, (n, k)).astype(np.int8)
    x = synth.activations(m, k, seed=m + k, dtype=torch.float32, outlier_p=0.01, outlier_mult=20.0).numpy()
    xq, a = oracle.quant_acts(x)
    gamma = np.float32(0.0159577)
    d = lambda arr: torch.from_numpy(arr).to(DEV)
    y, acc = bl.forward(d(oracle.pack(q)), d(np.array([gamma], np.float32)), d(xq), d(a), n, k,
                        want_y=True, want_acc=True)
    torch.cuda.synchronize()
    acc_ref, y_ref = oracle_forward_rows(q, gamma, xq, a, k)
    check_equal(host(acc), acc_ref, f"acc m={m} n={n} k={k}")
    check_y(host(y), y_ref, f"y m={m} n={n} k={k}")


def test_forward_extreme_accumulators():
    # all +1 / all -1 rows against all +127 activations: |acc| = 127 K, the int32 range
    # the path guarantees for the largest K of the workloads
    k = 28672
    for m in (1, 16, 40, 80):
        _announce("forward extreme", m)
        q = np.ones((32, k), np.int8)
        q[1::2] = -1
        xq = np.full((m, k), 127, np.int8)
        a = np.full(m, 127.0, np.float32)
        d = lambda arr: torch.from_numpy(arr).to(DEV)
        y, acc = bl.forward(d(oracle.pack(q)), d(np.array([1.0], np.float32)), d(xq), d(a), 32, k,
                            want_y=True, want_acc=True)
        torch.cuda.synchronize()
        exp = np.tile(np.array([127 * k, -127 * k], np.int64), 16)
        assert np.array_equal(host(acc), np.broadcast_to(exp, (m, 32)))
        check_y(host(y), np.broadcast_to(exp.astype(np.float64), (m, 32)), "extreme y")


@pytest.mark.parametrize("m", [1, 3, 17])
def test_forward_at_the_largest_k(m):
    # K = 2^24, the library's limit: |acc| <= 127 K = 2^31 - 2^24 still fits int32.  Closed
    # form on extreme rows (all +1 / all -1 against +127), and random codes against the
    # oracle on the decode kernels (M = 1, 3; M = 17 in two token groups).  The prefill kernel
    # meets the same per-element bound at K = 28672 in test_forward_extreme_accumulators.
    k, n = 1 << 24, 18
    _announce("forward at K = 2^24", m)
    rng = np.random.default_rng(m)
    q = rng.integers(-1, 2, (n, k)).astype(np.int8)
    q[0] = 1
    q[1] = -1
    xq = rng.integers(-127, 128, (m, k)).astype(np.int8)
    xq[0] = 127
    a = rng.uniform(0.5, 2.0, m).astype(np.float32)
    d = lambda arr: torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)
    y, acc = bl.forward(d(oracle.pack(q)), d(np.array([0.01], np.float32)), d(xq), d(a), n, k,
                        want_y=True, want_acc=True)
    torch.cuda.synchronize()
    acc_ref, y_ref = oracle.forward(q, np.float32(0.01), xq, a, k)
    assert acc_ref[0, 0] == 127 * k and acc_ref[0, 1] == -127 * k
    check_equal(host(acc), acc_ref, f"acc K=2^24 m={m}")
    check_y(host(y), y_ref, f"y K=2^24 m={m}")


def test_forward_only_acc_or_only_y():
    m, n, k = 3, 40, 512
    rng = np.random.default_rng(1)
    q = rng.integers(-1, 2, (n, k)).astype(np.int8)
    xq = rng.integers(-127, 128, (m, k)).astype(np.int8)
    a = np.ones(m, np.float32)
    d = lambda arr: torch.from_numpy(arr).to(DEV)
    acc = bl.forward(d(oracle.pack(q)), d(np.array([0.5], np.float32)), d(xq), d(a), n, k, want_y=False,
                     want_acc=True)
    y = bl.forward(d(oracle.pack(q)), d(np.array([0.5], np.float32)), d(xq), d(a), n, k)
    torch.cuda.synchronize()
    acc_ref = oracle.matmul(q, xq, k)
    check_equal(host(acc), acc_ref, "acc only")
    check_y(host(y), oracle.rescale(acc_ref, np.float32(0.5), a), "y only")


def test_forward_deterministic():
    n, k = 2560, 6912
    for m in (1, 16, 300):
        w = synth.latent_weights(n, k, seed=5, device=DEV)
        packed, gamma = bl.quantize_weights(w)
        xq, a = bl.quantize_acts(synth.activations(m, k, seed=6, device=DEV))
        r1 = bl.forward(packed, gamma, xq, a, n, k, want_acc=True)
        r2 = bl.forward(packed, gamma, xq, a, n, k, want_acc=True)
        torch.cuda.synchronize()
        assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


def test_binding_errors_are_raised():
    w = torch.zeros(4, 4, device=DEV, dtype=torch.float16)
    with pytest.raises(ValueError):
        bl.quantize_weights(w)
    xq = torch.zeros((1, 256), dtype=torch.int8, device=DEV)
    a = torch.zeros(1, dtype=torch.float32, device=DEV)
    g = torch.zeros(1, dtype=torch.float32, device=DEV)
    packed = torch.zeros(bl.packed_bytes(16, 256) + 16, dtype=torch.uint8, device=DEV)[8:]  # misaligned
    with pytest.raises(bl.BitLinearError):
        bl.forward(packed, g, xq, a, 16, 256)


# ------------------------------------------------------------------ fused quantise + forward
def _fused_check(m, n, k, dtype, seed, unaligned=False):
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, (n, k)).astype(np.int8)
    packed = torch.from_numpy(oracle.pack(q)).to(DEV)
    if unaligned:
        flat = synth.activations(1, m * k + 1, seed=seed, dtype=dtype, device=DEV,
                                 outlier_p=0.01, outlier_mult=20.0).reshape(-1)
        x = flat[1:].view(m, k)
    else:
        x = synth.activations(m, k, seed=seed, dtype=dtype, device=DEV, outlier_p=0.01, outlier_mult=20.0)
    if m > 2:
        x[1] = 0
    gamma = np.float32(0.0159577)
    (y, acc), xq, a = bl.forward_fused(packed, torch.tensor([gamma], device=DEV), x, n, k, want_y=True, want_acc=True)
    torch.cuda.synchronize()
    xq_ref, a_ref = oracle.quant_acts(acts_host_f32(x))
    check_equal(host(xq), xq_ref, f"fused xq m={m} k={k}")
    check_equal(host(a).view(np.uint32), a_ref.view(np.uint32), f"fused absmax m={m} k={k}")
    acc_ref, y_ref = oracle.forward(q, gamma, xq_ref, a_ref, k)
    check_equal(host(acc), acc_ref, f"fused acc m={m} n={n} k={k}")
    check_y(host(y), y_ref, f"fused y m={m} n={n} k={k}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("m,n,k", [(1, 512, 256), (1, 700, 2560), (2, 130, 4096), (3, 48, 1000), (4, 520, 2048),
                                   (1, 33, 8), (1, 16400, 512), (1, 64, 6912), (2, 130, 6912), (1, 40, 30000),
                                   (2, 100, 12000), (4, 24, 4096),
                                   # 257..512 row blocks, runs of at most 4 tiles: weights issued
                                   # once the activations land; 513 blocks: after the barrier
                                   (2, 6912, 2560), (4, 8192, 4096), (3, 4100, 1000), (1, 8192, 8192),
                                   (1, 8208, 2560)])
def test_forward_fused_single_kernel(m, n, k, dtype):
    # shapes one fused kernel takes: activation pieces held in registers, per-token absmax
    # across the workgroup's waves, ragged K, one to four tokens
    plan = bl.forward_fused_plan(m, n, k, "bf16" if dtype == torch.bfloat16 else "f32")
    _announce("forward fused", m, n, k, dtype, plan)
    assert plan["kernel"] == "fused" and plan["acts"] == "registers"
    _fused_check(m, n, k, dtype, seed=m * 31 + n + k)


@pytest.mark.parametrize("m,n,k,dtype", [(5, 512, 256, torch.bfloat16), (8, 700, 2560, torch.bfloat16),
                                         (9, 130, 4096, torch.bfloat16), (16, 6912, 2560, torch.bfloat16),
                                         (12, 640, 2560, torch.bfloat16), (16, 33, 8, torch.bfloat16),
                                         (7, 100, 1000, torch.bfloat16), (15, 1000, 3000, torch.bfloat16),
                                         (16, 8208, 2560, torch.bfloat16), (8, 700, 2560, torch.float32),
                                         (16, 2560, 6912, torch.bfloat16), (16, 2560, 2048, torch.bfloat16),
                                         (6, 1000, 4104, torch.bfloat16), (16, 520, 4096, torch.bfloat16),
                                         (11, 300, 4088, torch.bfloat16), (16, 11000, 1024, torch.bfloat16),
                                         (8, 2560, 6912, torch.bfloat16), (9, 700, 7168, torch.bfloat16),
                                         (5, 520, 7176, torch.bfloat16), (7, 2000, 5000, torch.bfloat16),
                                         (5, 1, 8, torch.bfloat16), (9, 1, 7168, torch.bfloat16),
                                         (16, 1, 7168, torch.bfloat16),
                                         (13, 6000, 2560, torch.bfloat16), (16, 300, 4097, torch.bfloat16)])
def test_forward_fused_5_to_16_tokens(m, n, k, dtype):
    # 5..16 tokens: one launch where every workgroup quantises the 16 token rows into LDS
    # (bf16 x, K a multiple of 8 up to 7168 and M K up to 64 Ki: eight waves of two rows; 1,
    # 2 or 4 row blocks per workgroup up to K = 4096); else the quantiser and the forward as
    # two launches inside the one call (ragged K and N, fp32 x, long rows)
    plan = bl.forward_fused_plan(m, n, k, "bf16" if dtype == torch.bfloat16 else "f32")
    _announce("forward fused 5..16", m, n, k, dtype, plan)
    one_launch = dtype == torch.bfloat16 and k % 8 == 0 and k <= 7168 and m * k <= 65536
    assert (plan["kernel"] == "fused" and plan["acts"] == "lds16") == one_launch, plan
    _fused_check(m, n, k, dtype, seed=m * 41 + n + k)


@pytest.mark.parametrize("m", [5, 16])
def test_forward_fused_5_to_16_nonfinite_rows(m):
    # rows holding a NaN (quiet, a signalling bit pattern, a negative one) or an infinity:
    # the one-launch 5..16-token form takes the absmax over the bit patterns of |x| and
    # falls back to the float maximum where a row holds a NaN.  The oracle's absmax passes
    # over NaN (a comparison with NaN is false) and an infinite absmax gives a zero scale;
    # the codes of the non-finite entries themselves are not defined by the oracle
    # (rounding NaN to an integer), so only the finite entries' codes are compared.
    n, k = 640, 2560
    plan = bl.forward_fused_plan(m, n, k, "bf16")
    _announce("forward fused 5..16 non-finite rows", m, n, k, plan)
    assert plan["kernel"] == "fused" and plan["acts"] == "lds16"
    q = np.random.default_rng(m).integers(-1, 2, (n, k)).astype(np.int8)
    packed = torch.from_numpy(oracle.pack(q)).to(DEV)
    x = synth.activations(m, k, seed=97 + m, dtype=torch.bfloat16, device=DEV, outlier_p=0.01, outlier_mult=20.0)
    bits = x.view(torch.int16)
    planted = [(0, 5, 0x7FC0), (1, k - 1, 0x7F81), (2, 100, 0xFFC0 - 0x10000), (3, 7, 0x7F80), (4, 9, 0xFF80 - 0x10000)]
    for r, c, b in planted:
        bits[r, c] = b
    bits[4, 10] = 0x7FC1  # a NaN beside the negative infinity
    (y, acc), xq, a = bl.forward_fused(packed, torch.tensor([0.02], device=DEV), x, n, k, want_y=True, want_acc=True)
    torch.cuda.synchronize()
    xf = acts_host_f32(x)
    xq_ref, a_ref = oracle.quant_acts(np.where(np.isfinite(xf), xf, 0.0).astype(np.float32))
    # the absmax over the row with its non-finite entries: NaN passes, infinity wins
    a_exp = a_ref.copy()
    for r in range(m):
        if np.isinf(xf[r]).any():
            a_exp[r] = np.inf
    check_equal(host(a).view(np.uint32), a_exp.view(np.uint32), f"absmax m={m}")
    finite = np.isfinite(xf)
    got = host(xq)[:, :k]
    for r in range(m):
        if np.isinf(a_exp[r]):
            # zero scale: every finite entry's code is 0
            assert (got[r][finite[r]] == 0).all(), r
        else:
            assert np.array_equal(got[r][finite[r]], xq_ref[r, :k][finite[r]]), r
    # rows without non-finite entries are unaffected: their outputs match the oracle
    clean = [r for r in range(m) if finite[r].all()]
    acc_ref, _ = oracle.forward(q, np.float32(0.02), xq_ref, a_ref, k)
    check_equal(host(acc)[clean], acc_ref[clean], f"acc of the finite rows m={m}")


@pytest.mark.parametrize("m,n,k,dtype", [(3, 65600, 768, torch.float32), (4, 70000, 1024, torch.float32)])
def test_forward_fused_lds_form(m, n, k, dtype):
    # many row blocks leave one wave per block; where its pieces would not fit in
    # registers, short rows are quantised into LDS by every workgroup instead
    plan = bl.forward_fused_plan(m, n, k, "bf16" if dtype == torch.bfloat16 else "f32")
    _announce("forward fused lds", m, n, k, dtype, plan)
    assert plan["kernel"] == "fused" and plan["acts"] == "lds"
    _fused_check(m, n, k, dtype, seed=m * 13 + n + k)


# One token on many row blocks (257 .. 1875, several workgroups per compute unit), ragged
# last rows (29999) and ragged K, int8 and fused: the 100B-class shapes and others.  Past
# 512 row blocks the fused form issues its activation loads at raised wave priority; up to
# 512 with runs of 14 or 16 tiles (8192 x 28672, 4200 x 32000, 6000 x 32504, 8100 x 28000
# with an odd number of row blocks, 7500 x 28504 with ragged K) it also issues two weight
# tiles ahead of the barrier.
MANY_RB = [(28672, 8192), (8192, 28672), (4100, 296), (16400, 296), (6912, 2560), (29999, 4000), (8200, 12000),
           (5000, 20000), (4200, 32000), (12288, 3000), (16000, 1104), (24576, 5000), (6000, 32504), (8100, 28000),
           (7500, 28504)]


@pytest.mark.parametrize("n,k", MANY_RB)
def test_forward_many_row_blocks(n, k):
    plan = bl.forward_plan(1, n, k)
    _announce("forward many row blocks", 1, n, k, plan)
    assert plan["kernel"] == "decode"
    _fwd_check(1, n, k, seed=n + 7 * k)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n,k", MANY_RB)
def test_forward_fused_many_row_blocks(n, k, dtype):
    plan = bl.forward_fused_plan(1, n, k, "bf16" if dtype == torch.bfloat16 else "f32")
    _announce("forward fused many row blocks", 1, n, k, dtype, plan)
    _fused_check(1, n, k, dtype, seed=n + 11 * k)


@pytest.mark.parametrize("m,n,k,dtype,unaligned", [(5, 64, 7176, torch.bfloat16, False), (1, 64, 300, torch.bfloat16, False),
                                                   (2, 64, 1002, torch.float32, False), (3, 40, 512, torch.bfloat16, True),
                                                   (40, 72, 700, torch.float32, False), (100, 72, 700, torch.bfloat16, False),
                                                   (3, 40, 12000, torch.float32, False),
                                                   (4, 30, 20000, torch.bfloat16, False)])
def test_forward_fused_fallback(m, n, k, dtype, unaligned):
    # shapes outside the one-kernel path: the quantiser kernel then the forward kernel
    plan = bl.forward_fused_plan(m, n, k, "bf16" if dtype == torch.bfloat16 else "f32")
    _announce("forward fused fallback", m, n, k, dtype, unaligned, plan)
    assert unaligned or plan["kernel"] != "fused"
    _fused_check(m, n, k, dtype, seed=m * 17 + n + k, unaligned=unaligned)


# ------------------------------------------------------------------ grouped projections
def _grouped_check(m, ns, k, dtype, seed):
    rng = np.random.default_rng(seed)
    qs = [rng.integers(-1, 2, (n, k)).astype(np.int8) for n in ns]
    gammas = [np.float32(0.01 + 0.001 * i) for i in range(len(ns))]
    x = synth.activations(m, k, seed=seed, dtype=dtype, device=DEV, outlier_p=0.01, outlier_mult=20.0)
    if m > 2:
        x[1] = 0
    mats = [(torch.from_numpy(oracle.pack(q)).to(DEV), torch.tensor([g], device=DEV), n)
            for q, g, n in zip(qs, gammas, ns)]
    outs, xq, a = bl.forward_grouped(mats, x, k, want_y=True, want_acc=True)
    torch.cuda.synchronize()
    xq_ref, a_ref = oracle.quant_acts(acts_host_f32(x))
    check_equal(host(xq), xq_ref, f"grouped xq m={m} k={k}")
    check_equal(host(a).view(np.uint32), a_ref.view(np.uint32), f"grouped absmax m={m} k={k}")
    for i, ((y, acc), q, g) in enumerate(zip(outs, qs, gammas)):
        acc_ref, y_ref = oracle.forward(q, g, xq_ref, a_ref, k)
        check_equal(host(acc), acc_ref, f"grouped acc {i} m={m} k={k}")
        check_y(host(y), y_ref, f"grouped y {i} m={m} k={k}")


@pytest.mark.parametrize("m,ns,k,dtype", [
    (1, [6912, 6912], 2560, torch.bfloat16),           # gate + up of a 2B-class layer
    (1, [2560, 640, 640], 2560, torch.bfloat16),       # Q, K, V
    (2, [17, 300, 1000], 1000, torch.float32),         # ragged rows and columns
    (3, [16, 33, 48, 64, 80, 96, 112, 130], 512, torch.bfloat16),  # eight matrices
    (4, [700, 900], 4096, torch.float32),
    (1, [512], 256, torch.float32),                    # a group of one
    (8, [300, 100], 2560, torch.bfloat16),             # more tokens: quantiser once, then one grouped forward
    (40, [130, 64], 1000, torch.float32),              # 17..64 tokens: token groups
    (100, [130, 64], 1000, torch.bfloat16),            # prefill sizes
    (1, [100, 200], 300, torch.bfloat16),              # K not a multiple of 8: quantiser path
    (2, [2560, 2560], 2560, torch.bfloat16),           # 320 row blocks: weights issued as activations land
    # 5..16 tokens, bf16: one launch that quantises into LDS in every workgroup
    (16, [2560, 640, 640], 2560, torch.bfloat16),      # Q, K, V of the 2B-class layer
    (16, [6912, 6912], 2560, torch.bfloat16),          # gate + up (864 row blocks: four per workgroup)
    (7, [33, 500, 17, 1000], 4096, torch.bfloat16),    # ragged rows, 16 K tiles, 7 tokens
    (8, [2560, 100], 6912, torch.bfloat16),            # 27 K tiles: runs of 4, one row block per workgroup
    (10, [4096, 4096, 100], 1000, torch.bfloat16),     # 520 row blocks: two per workgroup
    # 5..16 tokens otherwise: the quantiser, then one launch of the 5..16-token decode
    (16, [2560], 6912, torch.bfloat16),                # down: long rows, one forward
    (5, [17, 300, 1000, 33], 1000, torch.float32),     # ragged rows and columns, token group of 8
    (12, [130, 2100], 3000, torch.bfloat16),           # token group of 16, ragged K
    (9, [16, 32, 48, 64, 80, 96, 112, 6150], 4096, torch.float32),  # eight matrices, 16 K tiles
    (16, [16, 33, 48, 700, 80, 96, 112, 6150], 4096, torch.bfloat16),  # eight matrices in the fused form, 2 row blocks per WG
    (9, [2000, 17, 4100], 7168, torch.bfloat16),       # the longest fused rows (28 K tiles), M K = 64512
    (5, [8200, 8], 8, torch.bfloat16),                 # K = 8: one K tile, mostly padding, 514 row blocks
    (16, [300, 500], 4097, torch.bfloat16),            # 17 K tiles: one forward per matrix
    (1, [4096, 2048], 4096, torch.float32),            # 384 row blocks
])
def test_forward_grouped(m, ns, k, dtype):
    _announce("forward grouped", m, ns, k, dtype)
    _grouped_check(m, ns, k, dtype, seed=m * 71 + sum(ns) + k)
