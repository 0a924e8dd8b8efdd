"""bitlinear_quantize_weights_noalloc, the weight quantiser for callers that cannot
allocate: called through the C ABI, its packed codes and gamma must equal those of
bitlinear_quantize_weights (which takes a caller workspace) bit for bit, on two calls in a
row on the same GPU, the second with a smaller input (the static scratch keeps the first
call's bins, so this also checks that every call clears them)."""
import numpy as np
import pytest
import torch

import bitlinear_fwd_amd as bl
from bitlinear_fwd_amd import synth
from gpu_helpers import check_equal, gamma_bits, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(n, k, seed):
    print(f"case: quantize_weights_noalloc N={n} K={k} seed={seed}", flush=True)
    w = synth.latent_weights(n, k, seed=seed, device=DEV)
    p_ref, g_ref = bl.quantize_weights(w)
    p_new, g_new = bl.quantize_weights_noalloc(w)
    torch.cuda.synchronize()
    check_equal(host(p_new), host(p_ref), f"packed N={n} K={k}")
    assert gamma_bits(host(g_new)) == gamma_bits(host(g_ref)), (n, k)


def test_noalloc_matches_workspace_form_twice_shrinking():
    _both(6912, 2560, seed=41)   # a 2B-class matrix
    _both(300, 777, seed=42)     # then a smaller, ragged one on the same scratch


def test_noalloc_ragged_and_tiny():
    for n, k, seed in ((1, 1, 43), (17, 300, 44), (4100, 1000, 45), (16, 256, 46)):
        _both(n, k, seed)


def test_noalloc_rejects_bad_arguments():
    w = torch.zeros((4, 8), dtype=torch.float32, device=DEV)
    packed = torch.empty(bl.packed_bytes(4, 8), dtype=torch.uint8, device=DEV)
    gamma = torch.empty(1, dtype=torch.float32, device=DEV)
    L = bl.lib()
    s = torch.cuda.current_stream().cuda_stream
    assert L.bitlinear_quantize_weights_noalloc(None, 4, 8, packed.data_ptr(), gamma.data_ptr(), s) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_quantize_weights_noalloc(w.data_ptr(), 0, 8, packed.data_ptr(), gamma.data_ptr(), s) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_quantize_weights_noalloc(w.data_ptr(), 1 << 21, 1 << 20, packed.data_ptr(), gamma.data_ptr(),
                                                s) == bl.BL_ERR_UNSUPPORTED
    assert L.bitlinear_quantize_weights_noalloc(w.data_ptr(), 4, 8, packed.data_ptr() + 1, gamma.data_ptr(),
                                                s) == bl.BL_ERR_INVALID_ARG
    torch.cuda.synchronize()
