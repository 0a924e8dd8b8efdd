"""The measurement probes behind the benchmark's ceilings: the stream probe reads every
byte it is given (its per-block XOR checksums match numpy's), and the MFMA probe runs
and is deterministic."""
import numpy as np
import pytest
import torch

import bitlinear_fwd_amd as bl
from gpu_helpers import host

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("nbytes", [1024, 32768, 33 * 32768 + 5 * 1024, 4_423_680])
def test_probe_stream_reads_every_word(nbytes):
    print(f"case: probe_stream {nbytes} B", flush=True)
    rng = np.random.default_rng(nbytes)
    data = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(data.view(np.uint8)).to(DEV)
    out = bl.probe_stream(buf)
    torch.cuda.synchronize()
    words_per_block = 32768 // 4
    blocks = (data.size + words_per_block - 1) // words_per_block
    ref = np.array([np.bitwise_xor.reduce(data[i * words_per_block:(i + 1) * words_per_block])
                    for i in range(blocks)], np.uint32)
    assert np.array_equal(host(out).view(np.uint32), ref)


def test_probe_mfma_runs_deterministically():
    print("case: probe_mfma", flush=True)
    a = torch.empty(64, dtype=torch.int32, device=DEV)
    b = torch.empty(64, dtype=torch.int32, device=DEV)
    bl.probe_mfma(100, 64, a)
    bl.probe_mfma(100, 64, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("nbytes,groups", [(16, 1), (4096, 3), (1_000_016, 7), (4_423_680, 2048), (58_720_256, 2048)])
@pytest.mark.parametrize("nontemporal", [True, False])
def test_probe_read_reads_every_word(nbytes, groups, nontemporal):
    # the plain grid-stride read: workgroup b's checksum is the XOR of the 16-byte words
    # j = 256 b + t + 256 G i (t = 0..255, i >= 0) it owns
    print(f"case: probe_read {nbytes} B, {groups} workgroups, nontemporal={nontemporal}", flush=True)
    rng = np.random.default_rng(nbytes + groups)
    data = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(data.view(np.uint8)).to(DEV)
    out = bl.probe_read(buf, groups, nontemporal)
    torch.cuda.synchronize()
    words16 = np.bitwise_xor.reduce(data.reshape(-1, 4), axis=1)  # XOR of each 16-byte word
    owner = (np.arange(words16.size) // 256) % groups
    ref = np.zeros(groups, np.uint32)
    np.bitwise_xor.at(ref, owner, words16)
    assert np.array_equal(host(out).view(np.uint32), ref)
