"""GPU parity of bitlinear_forward_ws (the prefill GEMM with a caller workspace) against the
CPU oracle, on every output.

Where the output tiles need more than one round of the resident workgroups, the call runs
the split-tail form: whole tiles first, then the tiles left over split along K into
ranges whose exact int32 partial tiles a second launch adds.  Each
case checks the plan (so the split tail really runs), then acc bit-exact and y within
1e-5 relative against the oracle on every row (rows split over host threads)."""
import numpy as np
import pytest
import torch

import bitlinear_fwd_amd as bl
import oracle
from bitlinear_fwd_amd import synth
from gpu_helpers import check_equal, check_y, host, oracle_forward_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _announce(*a):
    print("case:", *a, flush=True)


def _inputs(m, n, k, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, (n, k)).astype(np.int8)
    x = synth.activations(m, k, seed=seed, dtype=torch.float32, outlier_p=0.01, outlier_mult=20.0).numpy()
    x[m // 3] = 0  # a zero token
    xq, a = oracle.quant_acts(x)
    return q, xq, a, np.float32(0.0159577)


def _run_ws(q, xq, a, gamma, n, k, ws):
    d = lambda arr: torch.from_numpy(arr).to(DEV)
    y, acc = bl.forward_ws(d(oracle.pack(q)), d(np.array([gamma], np.float32)), d(xq), d(a), n, k, workspace=ws,
                           want_y=True, want_acc=True)
    torch.cuda.synchronize()
    return host(y), host(acc)


# (M, N, K, tile_n, split tiles, K ranges): M, N and K ragged against the 64-row tiles and
# the 256-column chunks; three to twelve K ranges per split tile.  Where the tiles take more
# than one round or 64 x 256 tiles would leave a tail, the planner now takes the eight-wave
# 64 x 384 tiles instead (no split), so every split it makes follows one round of 64 x 192
# tiles.
SPLIT_CASES = [
    (1600, 8000, 1000, 192, 26, 4),     # 1050 tiles of 64 x 192: one round, 26 tiles in 4 ranges
    (4721, 2600, 3001, 192, 12, 12),    # 12 ranges of one chunk, K ragged
    (2961, 4100, 2560, 192, 10, 10),    # 10 tiles in 10 ranges
    (1037, 12000, 700, 192, 47, 3),     # 47 tiles in 3 ranges (K ragged)
    (614, 19968, 700, 192, 16, 3),      # 1040 tiles from ten 64-row blocks: 16 tiles in 3 ranges
]


@pytest.mark.parametrize("m,n,k,tile_n,tail,parts", SPLIT_CASES)
def test_forward_ws_split_tail(m, n, k, tile_n, tail, parts):
    plan = bl.forward_ws_plan(m, n, k)
    _announce("forward_ws split tail", m, n, k, plan)
    assert plan.get("split_tail") and plan["tile_n"] == tile_n == bl.forward_plan(m, n, k)["tile_n"]
    assert plan["split_tiles"] == tail and plan["k_ranges"] == parts
    q, xq, a, gamma = _inputs(m, n, k, seed=m + n + k)
    ws = torch.full((bl.forward_ws_bytes(m, n, k),), 0xA5, dtype=torch.uint8, device=DEV)  # no zeroing needed
    y, acc = _run_ws(q, xq, a, gamma, n, k, ws)
    acc_ref, y_ref = oracle_forward_rows(q, gamma, xq, a, k)
    check_equal(acc, acc_ref, f"acc m={m} n={n} k={k}")
    check_y(y, y_ref, f"y m={m} n={n} k={k}")


def test_forward_ws_reuses_workspace():
    # one workspace, three calls of different shapes in a row on one stream (the second
    # smaller, the third with no split), filled with garbage first: nothing in it carries
    # over from one call to the next
    shapes = [(4721, 2600, 3001), (1600, 8000, 1000), (300, 1000, 700)]
    ws = torch.randint(0, 256, (max(bl.forward_ws_bytes(*s) for s in shapes),), dtype=torch.uint8, device=DEV)
    for (m, n, k) in shapes:
        plan = bl.forward_ws_plan(m, n, k)
        _announce("forward_ws reuse", m, n, k, plan)
        q, xq, a, gamma = _inputs(m, n, k, seed=7 * m + k)
        y, acc = _run_ws(q, xq, a, gamma, n, k, ws)
        acc_ref, y_ref = oracle_forward_rows(q, gamma, xq, a, k)
        check_equal(acc, acc_ref, f"acc m={m} n={n} k={k}")
        check_y(y, y_ref, f"y m={m} n={n} k={k}")


@pytest.mark.parametrize("m,n,k", [(300, 1000, 700), (2048, 2560, 6912), (2048, 6912, 2560), (8, 512, 256)])
def test_forward_ws_without_split(m, n, k):
    # shapes whose plan splits nothing need no workspace: the call is bitlinear_forward
    # (2048 x 6912 x 2560 has a partial last round, but its partial tiles would exceed the
    # planner's 8 MiB)
    assert bl.forward_ws_bytes(m, n, k) == 0
    _announce("forward_ws no split", m, n, k, bl.forward_ws_plan(m, n, k))
    q, xq, a, gamma = _inputs(m, n, k, seed=m * 3 + n)
    y, acc = _run_ws(q, xq, a, gamma, n, k, None)
    acc_ref, y_ref = oracle_forward_rows(q, gamma, xq, a, k)
    check_equal(acc, acc_ref, f"acc m={m} n={n} k={k}")
    check_y(y, y_ref, f"y m={m} n={n} k={k}")


def test_forward_ws_rejects_small_workspace():
    m, n, k = 1600, 8000, 1000
    need = bl.forward_ws_bytes(m, n, k)
    ws = torch.zeros(need - 256, dtype=torch.uint8, device=DEV)
    xq = torch.zeros((m, k), dtype=torch.int8, device=DEV)
    a = torch.ones(m, device=DEV)
    packed = torch.zeros(bl.packed_bytes(n, k), dtype=torch.uint8, device=DEV)
    g = torch.ones(1, device=DEV)
    with pytest.raises(bl.BitLinearError):
        bl.forward_ws(packed, g, xq, a, n, k, workspace=ws)
    with pytest.raises(bl.BitLinearError):
        bl.forward_ws(packed, g, xq, a, n, k, workspace=None)


def test_gemm_slots_per_cu_match_occupancy():
    # the planner's resident workgroups per compute unit for the one-group prefill kernels
    # agree with what the runtime reports for the built kernels
    occ = bl.prefill_occupancy()
    assert occ == {"whole": {256: 3, 192: 4}, "split": {256: 3, 192: 4}}, occ
