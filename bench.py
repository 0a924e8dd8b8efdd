"""Benchmark of the BitLinear forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload 4] [--legs 1,3,4i,...] [--prefill-shapes MxKxN,...]
                    [--graph] [--no-cpu-baseline] [--copy-calibration MIB]

A step is one pass of the hot path over one batch of synthetic input: for every matrix of
the workload, the per-token int8 activation quantiser and the forward (packed-ternary x
int8 contraction, exact int32 accumulation, fp32 rescale).  For a few tokens with short
rows the two run as one fused kernel (bitlinear_forward_fused); otherwise as two kernels.
Weights are quantised and packed once, before timing, as at model load.  Each step's
launches are C-ABI calls whose arguments were marshalled beforehand (one foreign call per
kernel, a microsecond or so of host time), so the host stays ahead of the GPU and the
timed region is the GPU's back-to-back execution.  --graph replays one captured HIP graph
per step instead; on this stack a graph adds about a microsecond per kernel node over
back-to-back stream launches, so it is the slower of the two for microsecond kernels.

Headline (default workload 4, M = 1): the 100B-class decode sweep, 8192 -> 28672 and
28672 -> 8192 over an 80-layer stack of distinct seeded weights (160 matrices, 9.4 GB of
packed weights, far beyond the 256 MB Infinity Cache, so every launch streams its weights
from HBM); this is the largest configuration that fits one GPU.  Exactly K steps are timed
after W warm-up steps, with a HIP event after every step on the stream the kernels run
on: value = packed-weight bytes per step / mean step time, in GB/s, and `trials` gives
the median, min and max of the K per-step times.  The JSON line also carries:
  roofline     the dominant kernel: algorithmic bytes (decode) or int8 ops (prefill) per
               launch / mean launch duration, against 8 TB/s or 5.0 POPS.  The duration
               comes from HIP events on the launch stream: the timed region over its
               launches when the step is nothing but that kernel, else passes of the
               forward launches alone.  traffic: measured HBM bytes per launch (see TRAFFIC);
  legs         the other workloads, each with at least 20 timed steps and 400 launches and
               its own per-step statistics; the 2B-class M = 1 decode ("1"), the 2048-token
               prefill ("3", int8 TOPS vs 5.0 POPS) and the int8-only decode of the
               headline matrices ("4i") carry their own roofline block.  Also: the M = 16
               2B-class layer ("2"), M = 8 on the headline matrices ("4"), the projections
               of one input grouped into one call ("1g", "2g"), the same workloads behind the
               sub-layer RMS normalisation ("1s", "1gs", "2s"), the gate/up pair with the
               squared-ReLU gating epilogue in one launch ("1f", "1fs"), the two-kernel int8
               path ("1i"), the table-lookup decode ("1l"), the 1-bit sign-binary variant
               ("1b", "4b"), and one GPU's share of the 100B-class matrices split over 8
               GPUs ("5");
  host_us_per_launch (config and each leg) the host's time to issue one launch inside the
               timed region: near the GPU's time per launch, the host sets the pace;
  gpu_state    rocm-smi clock and power readings before and after the timed region;
  quantisers   the weight quantiser (2560 -> 6912 fp32 latents) and the activation quantiser
               (bf16, decode and prefill sizes) timed alone, in bytes moved per second;
  ceilings     measured on this GPU: a plain grid-stride HBM read (no access pattern of the
               BitLinear kernels) at 58.7 MB and 4.4 MB per launch and at 1 GiB, the same
               sizes read with the decode kernels' tile pattern, and the int8 MFMA rate;
               roofline.frac_of_measured_ceiling sets the dominant kernel against the
               plain read of its launch size;
  cpu_baseline the CPU oracle on the host cores, on the same workload: all physical cores of
               this process's CPU set, each matrix's output rows split over them
               (cpu_baseline), and one thread on 2 of the 80 layers, scaled to the sweep
               (cpu_baseline_single_thread); with the CPU model, core counts and the
               oracle's compile flags.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
I8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA (no sparsity)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, choices=[0, 1, 2, 3, 4, 5])
    ap.add_argument("--legs", default="1,1g,1s,1gs,1f,1fs,1i,1l,1b,2,2g,2s,3,4,4i,4b,5",
                    help="other workloads timed into 'legs' ('' for none); a trailing g times the workload "
                         "with the projections of one input grouped into one call")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph instead of pre-marshalled eager launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="wall-clock budget of the all-cores oracle run (the single-thread run takes 2 layers)")
    ap.add_argument("--path", default="fused", choices=["fused", "int8"],
                    help="headline path: the fused quantise + decode kernel where the library fuses the shape "
                         "(default), or the activation quantiser then the int8 forward")
    ap.add_argument("--skip-ceilings", action="store_true",
                    help="profiling runs only: no probe ceilings and no quantiser timings (shorter traces); "
                         "frac_of_measured_ceiling is then omitted")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device three times (the reference kernel of "
                         "known size for scaling FETCH_SIZE / WRITE_SIZE counter runs)")
    ap.add_argument("--prefill-shapes", default="", metavar="MxKxN,...",
                    help="also time bitlinear_forward alone on these prefill shapes (tokens x in x out; "
                         "seeded synthetic inputs as the 2048-token workload's) and report them apart "
                         "from the legs")
    return ap.parse_args()


class Matrix:
    """One quantised weight matrix with its pre-drawn activations."""

    def __init__(self, bl, synth, wl, layer, midx, k, n, m, dev, binary=False, weights=None):
        if weights is not None:  # the same seeded weights, already quantised for another M
            self.packed, self.gamma = weights.packed, weights.gamma
        else:
            w = synth.latent_weights(n, k, seed=synth.weight_seed(wl.index, layer, midx), device=dev)
            self.packed, self.gamma = bl.quantize_weights_binary(w) if binary else bl.quantize_weights(w)
            del w
        self.x = synth.activations(m, k, seed=synth.act_seed(wl.index, layer, midx), dtype=wl.act_dtype,
                                   device=dev, outlier_p=wl.outlier_p, outlier_mult=wl.outlier_mult)
        self.n, self.k, self.m = n, k, m
        self.bytes = bl.packed_bytes_binary(n, k) if binary else bl.packed_bytes(n, k)
        self.ops = 2 * m * n * k


SUBLN_EPS = 1e-5


class Workload:
    def __init__(self, bl, synth, idx, m, dev, subln=False, path="fused", weights_from=None):
        import torch

        self.wl = synth.WORKLOADS[idx]
        self.m = m
        self.bl = bl
        self.subln = subln  # sub-layer RMS normalisation (per-matrix gain) in front of the quantiser
        # "fused": one call per matrix where the library fuses it; "int8": the quantiser, then
        # bitlinear_forward; "lut": the quantiser, then the table-lookup forward; "binary":
        # 1-bit sign-binary weights, the quantiser, then bitlinear_forward_binary
        self.path = path
        self.sweep = self.wl.layers > 1  # a step sweeps every layer instead of one set
        nsets = self.wl.layers if self.sweep else self.wl.rotate_sets
        share = weights_from is not None and weights_from.wl.index == idx and path != "binary" and \
            weights_from.path != "binary"
        self.sets = [[Matrix(bl, synth, self.wl, s, i, k, n, m, dev, binary=path == "binary",
                             weights=weights_from.sets[s][i] if share else None)
                      for i, (_, k, n) in enumerate(self.wl.matrices)] for s in range(nsets)]
        for s, st in enumerate(self.sets):
            for i, mat in enumerate(st):
                mat.gain = synth.subln_gain(mat.k, synth.gain_seed(idx, s, i), device=dev) if subln else None
        torch.cuda.synchronize()
        self.bufs = {}
        for mat in self.sets[0]:
            key = (mat.k, mat.n)
            if key not in self.bufs:
                self.bufs[key] = (torch.empty((m, bl.k_pad(mat.k)), dtype=torch.int8, device=dev),
                                  torch.empty(m, dtype=torch.float32, device=dev),
                                  torch.empty((m, mat.n), dtype=torch.float32, device=dev))
        # forward_fused for a few tokens (one kernel when the library fuses the shape, else
        # quantiser + forward); quantiser + forward otherwise
        self.use_fused = m <= 4 and path == "fused"
        plan = bl.forward_subln_plan if subln else bl.forward_fused_plan
        self.fused = {key: self.use_fused and plan(m, key[1], key[0], self._dt())["kernel"] == "fused"
                      for key in self.bufs}
        self.cursor = 0
        self.graphs = None
        self.calls = [self.prepared(group, False) for group in self.step_groups()]

    def _dt(self):
        import torch

        return "bf16" if self.wl.act_dtype == torch.bfloat16 else "f32"

    def step_groups(self):
        """The matrix lists of the distinct steps (one per weight set, or one sweep)."""
        return [sum(self.sets, [])] if self.sweep else self.sets

    def launch(self, mat, forward_only=False):
        bl = self.bl
        xq, a, y = self.bufs[(mat.k, mat.n)]
        if self.fused[(mat.k, mat.n)] or (self.use_fused and not forward_only):
            if self.subln:
                bl.forward_subln(mat.packed, mat.gamma, mat.x, mat.n, mat.k, mat.gain, SUBLN_EPS, y=y, xq=xq, scale=a)
            else:
                bl.forward_fused(mat.packed, mat.gamma, mat.x, mat.n, mat.k, y=y, xq=xq, absmax=a)
        else:
            if not forward_only:
                if self.subln:
                    bl.subln_quantize_acts(mat.x, mat.gain, SUBLN_EPS, xq, a)
                else:
                    bl.quantize_acts(mat.x, xq, a)
            if self.path == "lut":
                bl.forward_lut(mat.packed, mat.gamma, xq, a, mat.n, mat.k, y=y)
            elif self.path == "binary":
                bl.forward_binary(mat.packed, mat.gamma, xq, a, mat.n, mat.k, y=y)
            else:
                bl.forward(mat.packed, mat.gamma, xq, a, mat.n, mat.k, y=y)

    def set_gated_pair(self):
        """Gate and up (matrices 0 and 1, one input) as one gated squared-ReLU call, then the
        down projection: two launches per step, with the same weight bytes as the three."""
        import torch

        self.gated = True
        self.gated_h = [torch.empty((self.m, st[0].n), dtype=torch.float32, device=st[0].x.device) for st in self.sets]
        self.calls = [self.prepared(group, False) for group in self.step_groups()]

    def set_grouping(self, grouping):
        """Projections of one input launched as one grouped call: ``grouping`` lists the
        matrix indices of each group (a group's matrices take the first one's input).
        Every matrix gets its own output buffer."""
        import torch

        self.grouping = grouping
        self.group_y = [[torch.empty((self.m, mat.n), dtype=torch.float32, device=mat.x.device) for mat in st]
                        for st in self.sets]
        self.calls = [self.prepared(group, False) for group in self.step_groups()]

    def prepared(self, group, forward_only):
        """The step's launches as pre-marshalled C-ABI calls (one foreign call each)."""
        bl = self.bl
        if getattr(self, "gated", False) and not forward_only:
            si = next(i for i, st in enumerate(self.sets) if st[0] is group[0])
            gate, up, down = group
            xq, a, _ = self.bufs[(gate.k, gate.n)]
            calls = [bl.prepare_forward_gated_relu2((gate.packed, gate.gamma), (up.packed, up.gamma), gate.x, gate.n,
                                                    gate.k, self.subln, gate.gain, SUBLN_EPS, self.gated_h[si], xq, a)]
            xq, a, y = self.bufs[(down.k, down.n)]
            if self.subln:
                calls.append(bl.prepare_forward_subln(down.packed, down.gamma, down.x, down.n, down.k, down.gain,
                                                      SUBLN_EPS, y, xq, a))
            else:
                calls.append(bl.prepare_forward_fused(down.packed, down.gamma, down.x, down.n, down.k, y, xq, a))
            return calls
        if getattr(self, "grouping", None) and not forward_only:
            si = next(i for i, st in enumerate(self.sets) if st[0] is group[0])
            calls = []
            for idxs in self.grouping:
                first = group[idxs[0]]
                xq, a, _ = self.bufs[(first.k, first.n)]
                mats = [(group[i].packed, group[i].gamma, group[i].n, self.group_y[si][i]) for i in idxs]
                if self.subln:
                    calls.append(bl.prepare_forward_grouped_subln(mats, first.x, first.k, first.gain, SUBLN_EPS,
                                                                  xq, a))
                elif len(idxs) == 1:
                    calls.append(bl.prepare_forward_fused(first.packed, first.gamma, first.x, first.n, first.k,
                                                          self.group_y[si][idxs[0]], xq, a))
                else:
                    calls.append(bl.prepare_forward_grouped(mats, first.x, first.k, xq, a))
            return calls
        calls = []
        for mat in group:
            xq, a, y = self.bufs[(mat.k, mat.n)]
            if self.fused[(mat.k, mat.n)] or (self.use_fused and not forward_only):
                if self.subln:
                    calls.append(bl.prepare_forward_subln(mat.packed, mat.gamma, mat.x, mat.n, mat.k, mat.gain,
                                                          SUBLN_EPS, y, xq, a))
                else:
                    calls.append(bl.prepare_forward_fused(mat.packed, mat.gamma, mat.x, mat.n, mat.k, y, xq, a))
            else:
                if not forward_only:
                    if self.subln:
                        calls.append(bl.prepare_subln_quantize_acts(mat.x, mat.gain, SUBLN_EPS, xq, a))
                    else:
                        calls.append(bl.prepare_quantize_acts(mat.x, xq, a))
                if self.path == "lut":
                    calls.append(bl.prepare_forward_lut(mat.packed, mat.gamma, xq, a, mat.n, mat.k, y))
                elif self.path == "binary":
                    calls.append(bl.prepare_forward_binary(mat.packed, mat.gamma, xq, a, mat.n, mat.k, y))
                else:
                    calls.append(bl.prepare_forward(mat.packed, mat.gamma, xq, a, mat.n, mat.k, y))
        return calls

    def capture(self):
        """Record each step group's launches into a HIP graph: the same calls the eager steps
        make (grouped and gated calls included), prepared inside the capture so that they
        record onto the capture stream."""
        import torch

        self.graphs = []
        for i, group in enumerate(self.step_groups()):
            for call in self.calls[i]:  # warm the kernels once outside capture
                call()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for call in self.prepared(group, False):
                    call()
            self.graphs.append(g)
        torch.cuda.synchronize()

    def run_step(self):
        groups = self.step_groups()
        i = self.cursor
        self.cursor = (self.cursor + 1) % len(groups)
        if self.graphs is not None:
            self.graphs[i].replay()
        else:
            for call in self.calls[i]:
                call()

    def bytes_per_step(self):
        return sum(mat.bytes for mat in self.step_groups()[0])

    def ops_per_step(self):
        return sum(mat.ops for mat in self.step_groups()[0])

    def allin_bytes_per_step(self):
        """Algorithmic bytes of the whole step: packed weights, the activation input (x in
        its dtype) and the fp32 outputs of every matrix."""
        xb = 2 if self._dt() == "bf16" else 4
        return sum(mat.bytes + mat.m * mat.k * xb + mat.m * mat.n * 4 for mat in self.step_groups()[0])

    def matrices_per_step(self):
        return len(self.step_groups()[0])


# HBM traffic per launch of the dominant kernel, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, averaged over the step's launches), each
# scaled by what the same counter reads for a device-to-device copy of known size run in the
# same process (--copy-calibration).  A figure holds only for the kernel source it was taken
# on: a hash of the kernel sources' code (comments and whitespace left out) is stored with
# it, and a mismatch reports null.
KERNEL_SOURCES = {
    "decode": ("bitlinear_fwd_amd/csrc/gemv.hip", "bitlinear_fwd_amd/csrc/decode_common.h",
               "bitlinear_fwd_amd/csrc/bl_internal.h"),
    "prefill": ("bitlinear_fwd_amd/csrc/gemm.hip", "bitlinear_fwd_amd/csrc/bl_internal.h"),
}
TRAFFIC = {
    # (workload, M, path): scaled bytes per launch (fetch + write), raw KiB per launch, source hash.
    # path: "fused" (quantise + decode in one kernel), "int8" (decode of quantised
    # activations), "prefill".  Copy calibration (256 MiB device copy): FETCH_SIZE read
    # 131083.8-131086.5 KiB (x1.99978-1.99982, taken per run), WRITE_SIZE 262144.0 KiB (x1.0).
    (4, 1, "fused"): {"bytes_per_launch": 59264290, "fetch_kib": 28895.23, "write_kib": 90.03, "sha": "9a60bae9175f079c"},
    (4, 1, "int8"): {"bytes_per_launch": 59032887, "fetch_kib": 28791.25, "write_kib": 72.00, "sha": "9a60bae9175f079c"},
    (1, 1, "fused"): {"bytes_per_launch": 4591156, "fetch_kib": 2229.34, "write_kib": 25.28, "sha": "9a60bae9175f079c"},
    (2, 16, "int8"): {"bytes_per_launch": 3160685, "fetch_kib": 1441.72, "write_kib": 203.43, "sha": "9a60bae9175f079c"},
    (3, 2048, "prefill"): {"bytes_per_launch": 103728584, "fetch_kib": 31708.16, "write_kib": 37888.14, "sha": "0b835e9f806c2790"},
}


def source_sha(kind: str) -> str:
    """Hash of the kernel sources' code: comments and whitespace are left out, so a change
    of wording keeps the measured figures while any change of code drops them."""
    import hashlib
    import re

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: int, m: int, path: str):
    kind = "prefill" if kernel.startswith("k_gemm") else "decode"
    rec = TRAFFIC.get((workload, m, "prefill" if kind == "prefill" else path))
    if rec is None:
        return None
    return rec["bytes_per_launch"] if rec["sha"] == source_sha(kind) else None


# Projections that share one input in a transformer layer, by matrix index of the workload:
# gate/up (2B decode, workload 1); Q/K/V and gate/up (2B layer, workload 2).
GROUPINGS = {1: [[0, 1], [2]], 2: [[0, 1, 2], [3], [4, 5], [6]]}


def copy_calibration(mib: int):
    import torch

    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def measure_quantisers(bl, synth, dev, reps: int = 20):
    """The two quantiser steps timed on their own (HIP events around back-to-back calls on
    pre-allocated buffers), as bytes moved per second: the weight quantiser (a-1 + a-2:
    the fp32 latents read, the packed codes written) on a 2B-class 2560 -> 6912 matrix, and
    the activation quantiser (a-3: x read, int8 codes and scales written) at decode and
    prefill sizes."""
    import torch

    out = {}
    n, k = 6912, 2560
    w = synth.latent_weights(n, k, seed=7, device=dev)
    packed = torch.empty(bl.packed_bytes(n, k), dtype=torch.uint8, device=dev)
    gamma = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(bl.wq_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
    call = lambda: bl.quantize_weights(w, packed, gamma, ws)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    moved = 4 * n * k + bl.packed_bytes(n, k)
    out["weight_quant_2560x6912"] = {"us": round(us, 2), "GBps": round(moved / (us * 1e-6) / 1e9, 1)}
    del w, packed, ws
    for m, kk in ((1, 2560), (16, 2560), (2048, 2560), (2048, 6912)):
        x = synth.activations(m, kk, seed=8, dtype=torch.bfloat16, device=dev)
        xq = torch.empty((m, bl.k_pad(kk)), dtype=torch.int8, device=dev)
        a = torch.empty(m, dtype=torch.float32, device=dev)
        pc = bl.prepare_quantize_acts(x, xq, a)
        pc()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            pc()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        moved = 2 * m * kk + m * bl.k_pad(kk) + 4 * m
        out[f"act_quant_M{m}_K{kk}_bf16"] = {"us": round(us, 2), "GBps": round(moved / (us * 1e-6) / 1e9, 1)}
    return out


def _time_calls(calls, reps: int, warm: int = 20) -> float:
    """Mean µs per call of back-to-back pre-marshalled launches, HIP events on the stream."""
    import torch

    for i in range(warm):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        calls[i % len(calls)]()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def measure_ceilings(bl, dev):
    """Measured ceilings on this GPU (library probes, back-to-back launches timed with HIP
    events; the buffers rotate through a 2 GiB pool, so every launch reads from HBM):
      * read_*: a plain grid-stride read (bitlinear_probe_read) with no access pattern of
        the BitLinear kernels, at 58.7 MB and 4.4 MB per launch (the decode matrices'
        sizes) and 1 GiB; workgroup counts and load kinds swept, the best kept;
      * stream_*: the same sizes read with the decode kernels' tile pattern
        (bitlinear_probe_stream);
      * mfma_int8_TOPS: independent int8 MFMAs with no memory traffic."""
    import torch

    pool_bytes = 2 << 30
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    pool.fill_(0x5A)
    stream = torch.cuda.current_stream().cuda_stream
    out, sweep = {}, {}
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    for name, nbytes in (("58.7MB", 58_720_256), ("4.4MB", 4_423_680), ("1GiB", 1 << 30)):
        copies = pool_bytes // nbytes
        reps = 400 if nbytes < 10_000_000 else (200 if nbytes < 100_000_000 else 12)
        best = None
        for nt in (1, 0):
            for groups in (1024, 2048, 4096, 8192):
                calls = [bl.PreparedCall("bitlinear_probe_read", pool.data_ptr() + i * nbytes, nbytes, groups, nt,
                                         sink.data_ptr(), stream) for i in range(copies)]
                us = _time_calls(calls, reps, warm=min(20, 2 * copies))
                gbs = nbytes / (us * 1e-6) / 1e9
                sweep[f"read_{name}_wg{groups}_{'nt' if nt else 'plain'}_GBps"] = round(gbs, 1)
                if best is None or us < best[0]:
                    best = (us, gbs, groups, nt)
        out[f"read_{name}_us"] = round(best[0], 3)
        out[f"read_{name}_GBps"] = round(best[1], 1)
        out[f"read_{name}_config"] = f"{best[2]} workgroups, {'non-temporal' if best[3] else 'ordinary'} loads"
        if nbytes < (1 << 30):
            words = int(bl.lib().bitlinear_probe_stream_words(nbytes))
            tsink = torch.empty(words, dtype=torch.int32, device=dev)
            calls = [bl.PreparedCall("bitlinear_probe_stream", pool.data_ptr() + i * nbytes, nbytes, tsink.data_ptr(),
                                     words, stream) for i in range(copies)]
            us = _time_calls(calls, reps)
            out[f"stream_{name}_us"] = round(us, 3)
            out[f"stream_{name}_GBps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    out["read_sweep"] = sweep
    del pool
    torch.cuda.empty_cache()
    # about 5 ms per launch; the first launch brings the clocks up, the best of three counts
    groups, iters = 512, 16000
    msink = torch.empty(groups, dtype=torch.int32, device=dev)
    best = 0.0
    for rep in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bl.probe_mfma(iters, groups, msink)
        e1.record()
        torch.cuda.synchronize()
        if rep:
            best = max(best, 2.0 * 16 * 16 * 64 * 16 * iters * groups * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    out["mfma_int8_TOPS"] = round(best, 1)
    return out


def read_ceiling(ceilings, launch_bytes: float) -> float:
    """The plain-read ceiling of the probe size nearest the launch's bytes."""
    return ceilings["read_58.7MB_GBps"] if launch_bytes >= 20e6 else ceilings["read_4.4MB_GBps"]


def dominant_kernel(w: Workload) -> str:
    """Name of the kernel that takes the step's time, as the launch plan picks it."""
    m = w.m
    key = max(w.bufs, key=lambda kn: kn[0] * kn[1])
    plan = w.bl.forward_plan(m, key[1], key[0])
    if plan["kernel"] == "prefill":
        groups = ", two K groups per tile" if plan["k_groups"] == 2 else ""
        return "k_gemm_mfma (prefill, %dx%d tiles%s)" % (plan["tile_m"], plan["tile_n"], groups)
    if w.fused[key] and w.subln:
        return "k_gemv_dpp_norm (sub-layer normalisation + activation quantise + decode, one kernel)"
    if w.fused[key]:
        fplan = w.bl.forward_fused_plan(m, key[1], key[0], w._dt())
        if fplan["acts"] == "registers":
            return "k_gemv_dpp (fused activation quantise + decode, activations in registers)"
        return "k_gemv_lds (fused activation quantise + decode, activations in LDS)"
    if plan["acts"] == "registers":
        if m > 4:
            return "k_gemv_dppm (decode, 5..16 tokens, activation registers shared by row blocks)"
        return "k_gemv_dpp (decode, activations broadcast across lanes)"
    return "k_gemv_lds (decode, activations in LDS)" if plan["lds_acts"] else "k_gemv_reg (decode)"


def gpu_state():
    """Clock and power readings of the first GPU from rocm-smi (a child process), as the
    tool prints them; None where it is missing or fails.  Context for the timings: the
    clocks vary with load and temperature."""
    import shutil
    import subprocess

    try:
        # The tool is a Python script: run it with this interpreter rather than through its
        # `env` line, so no process in the chain replaces itself (a profiler's preloaded
        # library has already opened the GPU in every child).
        smi = os.path.realpath(shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi")
        out = subprocess.run([sys.executable, smi, "--showclocks", "--showpower", "--json"], capture_output=True,
                             text=True, timeout=20)
        card = next(iter(json.loads(out.stdout).values()))
        keep = ("sclk", "mclk", "fclk", "socclk", "power")
        return {k: v for k, v in card.items() if any(t in k.lower() for t in keep)}
    except Exception:
        return None


def time_steps(w: Workload, steps: int, warmup: int):
    """W untimed warm-up steps, then exactly `steps` timed steps with a HIP event recorded
    after each on the stream the kernels run on.  Returns (mean ms per step over the whole
    timed region, the per-step times in ms, the host's ms per step spent issuing them: where
    that reaches the GPU's time the launches, not the kernels, set the pace)."""
    import torch

    for _ in range(warmup):
        w.run_step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    t0 = time.perf_counter()
    for i in range(steps):
        w.run_step()
        ev[i + 1].record(stream)
    host_ms = (time.perf_counter() - t0) * 1e3 / steps
    torch.cuda.synchronize()
    trials = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, trials, host_ms


def trial_stats(trials, bytes_per_step=None, ops_per_step=None):
    """Median, min, max and mean of per-step times, and the rates at the median and the min."""
    import statistics

    med, lo = statistics.median(trials), min(trials)
    out = {"n": len(trials), "median_ms": round(med, 5), "min_ms": round(lo, 5), "max_ms": round(max(trials), 5),
           "mean_ms": round(sum(trials) / len(trials), 5)}
    if bytes_per_step:
        out["GBps_at_median"] = round(bytes_per_step / (med * 1e-3) / 1e9, 1)
        out["GBps_at_min"] = round(bytes_per_step / (lo * 1e-3) / 1e9, 1)
    if ops_per_step:
        out["TOPS_at_median"] = round(ops_per_step / (med * 1e-3) / 1e12, 2)
        out["TOPS_at_min"] = round(ops_per_step / (lo * 1e-3) / 1e12, 2)
    return out


def leg_steps(w: Workload, floor_steps: int = 20, floor_launches: int = 400):
    """Timed steps of a leg: at least 20 (the trial count) and at least 400 launches."""
    launches = max(1, len(w.calls[0]))
    return max(floor_steps, -(-floor_launches // launches))


def time_forward_only(w: Workload, reps: int):
    """Mean duration of one forward-kernel launch: HIP events on the stream the kernels run
    on, around `reps` passes over the step groups that issue only the forward launches
    (activations quantised beforehand where the step uses two kernels), launched the way
    the timed steps are (pre-marshalled eager calls, or graph replays)."""
    import torch

    groups = w.step_groups()
    for group in groups:
        for mat in group:
            w.launch(mat)  # leaves each matrix's quantised activations in place
    torch.cuda.synchronize()
    if w.graphs is not None:
        runs = []
        for group in groups:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for mat in group:
                    w.launch(mat, forward_only=True)
            runs.append(g.replay)
        keep = runs
    else:
        keep = [w.prepared(group, True) for group in groups]
        runs = [(lambda calls=calls: [c() for c in calls]) for calls in keep]
    for _ in range(3):  # warm: caches, and the clock out of its idle state
        for r in runs:
            r()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for r in range(reps):
        runs[r % len(runs)]()
    stop.record(stream)
    torch.cuda.synchronize()
    mats = [mat for r in range(reps) for mat in groups[r % len(groups)]]
    del keep, runs
    return (start.elapsed_time(stop) / len(mats), sum(m.bytes for m in mats) / len(mats),
            sum(m.ops for m in mats) / len(mats))


def time_prefill_shapes(bl, synth, dev, spec: str, reps: int = 40):
    """bitlinear_forward alone on each M x K x N of `spec`: the plan's tile, and the launch
    time as the fastest and the median of five windows of `reps` back-to-back launches (HIP
    events on the kernels' stream), with the int8 TOPS and the fraction of the 5 POPS peak."""
    import statistics

    import torch

    out = {}
    wl = synth.WORKLOADS[3]
    for tok in [t for t in spec.split(",") if t.strip()]:
        m, k, n = (int(v) for v in tok.lower().split("x"))
        w = synth.latent_weights(n, k, seed=synth.weight_seed(3, 90, 0), device=dev)
        packed, gamma = bl.quantize_weights(w)
        del w
        x = synth.activations(m, k, seed=synth.act_seed(3, 90, 0), dtype=wl.act_dtype, device=dev,
                              outlier_p=wl.outlier_p, outlier_mult=wl.outlier_mult)
        xq, a = bl.quantize_acts(x)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        call = bl.prepare_forward(packed, gamma, xq, a, n, k, y)
        for _ in range(10):
            call()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        wins = []
        for _ in range(5):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            for _ in range(reps):
                call()
            e.record(stream)
            torch.cuda.synchronize()
            wins.append(s.elapsed_time(e) * 1e3 / reps)
        med, lo = statistics.median(wins), min(wins)
        plan = bl.forward_plan(m, n, k)
        ops = 2 * m * n * k
        out[tok] = {"tile": f"{plan.get('tile_m')}x{plan.get('tile_n')}", "k_groups": plan.get("k_groups"),
                    "threads": plan.get("threads"), "launch_us_median": round(med, 3), "launch_us_min": round(lo, 3),
                    "TOPS_at_median": round(ops / (med * 1e-6) / 1e12, 2),
                    "mfma_frac_at_median": round(ops / (med * 1e-6) / 1e12 / I8_PEAK_TOPS, 4)}
        progress(f"prefill shape {tok}: {med:.2f} us per launch")
        del packed, gamma, x, xq, a, y, call
        torch.cuda.empty_cache()
    return out


def host_cpu_facts():
    """The host the oracle baseline runs on: CPU model, logical CPUs of the machine and of
    this process's CPU set, and the physical cores in that set (distinct (package, core)
    pairs of sysfs topology; hyper-threads of one core count once)."""
    aff = sorted(os.sched_getaffinity(0))
    cores = set()
    for c in aff:
        try:
            with open(f"/sys/devices/system/cpu/cpu{c}/topology/physical_package_id") as f:
                pkg = f.read().strip()
            with open(f"/sys/devices/system/cpu/cpu{c}/topology/core_id") as f:
                core = f.read().strip()
            cores.add((pkg, core))
        except OSError:
            cores.add(("cpu", c))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_in_affinity": len(aff),
            "physical_cores_in_affinity": len(cores)}


def _acts_host_f32(x):
    import numpy as np
    import torch

    import oracle

    if x.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f32(x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return x.float().cpu().numpy()


def cpu_baseline_single(w: Workload, layers: int = 2):
    """The oracle on one host thread over the matrices of the first `layers` layers of the
    step (weight sets, for a one-set step): act quant, unpack, integer matmul and rescale
    per matrix.  Returns (bytes, ops, seconds, matrices, matrices per step)."""
    import numpy as np

    import oracle

    mats = sum(w.sets[:layers], [])
    done_bytes = done_ops = 0
    t_used = 0.0
    for mat in mats:
        packed = mat.packed.cpu().numpy()
        x = _acts_host_f32(mat.x)
        g = np.float32(mat.gamma.cpu().numpy()[0])
        t0 = time.perf_counter()
        xq, a = oracle.quant_acts(x)
        q = oracle.unpack(packed, mat.n, mat.k)
        oracle.forward(q, g, xq, a, mat.k)
        t_used += time.perf_counter() - t0
        done_bytes += mat.bytes
        done_ops += mat.ops
    return done_bytes, done_ops, t_used, len(mats), w.matrices_per_step()


def cpu_baseline_cores(w: Workload, budget_s: float, threads: int):
    """The oracle on `threads` host threads over the step's matrices in order, until the
    wall-clock budget is spent or the step is done.  For each matrix the activation
    quantiser runs once; then the 16-row blocks of the output rows are split into
    `threads` contiguous slices, and each thread unpacks its slice of the packed bytes (a
    row block is a contiguous byte range) and computes its columns of the output (the
    oracle's C routines run outside the interpreter lock).  Host copies of the inputs are
    made outside the timed part.  Returns (bytes, ops, seconds, matrices, matrices per step)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    mats = w.step_groups()[0]
    done_bytes = done_ops = 0
    t_used = 0.0
    n_done = 0
    with ThreadPoolExecutor(threads) as pool:
        for mat in mats:
            if t_used >= budget_s:
                break
            packed = mat.packed.cpu().numpy()
            x = _acts_host_f32(mat.x)
            g = np.float32(mat.gamma.cpu().numpy()[0])
            blocks = -(-mat.n // 16)
            cuts = [blocks * i // threads for i in range(threads + 1)]

            def part(i, xq, a, packed=packed, mat=mat, g=g, cuts=cuts):
                lo, hi = cuts[i], cuts[i + 1]
                if lo == hi:
                    return None
                rows = min(mat.n, 16 * hi) - 16 * lo
                sub = packed[oracle.packed_bytes(16 * lo, mat.k):oracle.packed_bytes(16 * hi, mat.k)]
                q = oracle.unpack(np.ascontiguousarray(sub), rows, mat.k)
                return oracle.forward(q, g, xq, a, mat.k)[1]

            t0 = time.perf_counter()
            xq, a = oracle.quant_acts(x)
            ys = [y for y in pool.map(lambda i: part(i, xq, a), range(threads)) if y is not None]
            np.concatenate(ys, axis=1)
            t_used += time.perf_counter() - t0
            done_bytes += mat.bytes
            done_ops += mat.ops
            n_done += 1
    return done_bytes, done_ops, t_used, n_done, len(mats)


def roofline_block(w: Workload, launch_ms, launch_bytes, launch_ops, launch_timing, workload_idx, ceilings):
    """The roofline of the step's dominant kernel: algorithmic bytes (decode, HBM-bound) or
    int8 ops (prefill, MFMA-bound) per launch over the mean launch duration."""
    kernel = dominant_kernel(w)
    fused = w.path == "fused" and all(w.fused.values())
    traffic = measured_traffic(kernel, workload_idx, w.m, "fused" if fused else "int8")
    if w.m <= 16:
        achieved = launch_bytes / (launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
                "launch_us": round(launch_ms * 1e3, 3), "launch_timing": launch_timing,
                "algorithmic_bytes_per_launch": int(launch_bytes),
                "note": "algorithmic bytes are the 2-bit packed weights; the information bound of ternary "
                        "codes, log2(3) bits per weight, is 79 % of them"}
        if ceilings:
            c = read_ceiling(ceilings, launch_bytes)
            roof["measured_ceiling"] = c
            roof["measured_ceiling_kind"] = "plain grid-stride HBM read of the same bytes per launch"
            roof["frac_of_measured_ceiling"] = round(achieved / c, 4)
    else:
        # int8 contraction: TOPS against the dense int8 MFMA peak (unit kept as the contract's)
        achieved = launch_ops / (launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": I8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(achieved / I8_PEAK_TOPS, 4), "traffic": traffic, "kernel": kernel,
                "launch_us": round(launch_ms * 1e3, 3), "launch_timing": launch_timing,
                "algorithmic_ops_per_launch": int(launch_ops)}
        if ceilings:
            roof["measured_ceiling"] = ceilings["mfma_int8_TOPS"]
            roof["measured_ceiling_kind"] = "independent int8 MFMAs, no memory traffic"
            roof["frac_of_measured_ceiling"] = round(achieved / ceilings["mfma_int8_TOPS"], 4)
    return roof


def launch_timing_of(w: Workload, ms: float):
    """Mean forward-launch duration: the timed region over its launches when the step holds
    nothing but the fused kernel, else passes of the forward launches alone."""
    mats = w.step_groups()[0]
    if all(w.fused.values()) and not getattr(w, "grouping", None) and not getattr(w, "gated", False):
        return (ms / len(mats), w.bytes_per_step() / len(mats), w.ops_per_step() / len(mats),
                "timed region / launches (the step is only this kernel)")
    reps = max(20, len(w.step_groups())) if w.sweep else max(400, 4 * len(w.sets))
    l_ms, l_b, l_o = time_forward_only(w, reps)
    return l_ms, l_b, l_o, "HIP events around back-to-back forward launches alone (activations quantised before)"


def leg_summary(w: Workload, ms: float, trials, launch_ms, launch_bytes, launch_ops, ceilings=None):
    gbs = w.bytes_per_step() / (ms * 1e-3) / 1e9
    tops = w.ops_per_step() / (ms * 1e-3) / 1e12
    out = {
        "workload": w.wl.name, "M": w.m, "ms_per_step": round(ms, 5),
        "us_per_matrix": round(ms * 1e3 / w.matrices_per_step(), 3),
        "packed_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "allin_GBps": round(w.allin_bytes_per_step() / (ms * 1e-3) / 1e9, 1),
        "int8_TOPS": round(tops, 2), "mfma_frac": round(tops / I8_PEAK_TOPS, 4),
        "tokens_per_s_eq": round(w.m / (ms * 1e-3), 1),  # every matrix of the step applied once per token
        "launches_per_step": len(w.calls[0]),
        "trials": trial_stats(trials, w.bytes_per_step(), w.ops_per_step() if w.m > 16 else None),
    }
    if launch_ms is not None:
        out["forward_launch_us"] = round(launch_ms * 1e3, 3)
        out["forward_launch_GBps"] = round(launch_bytes / (launch_ms * 1e-3) / 1e9, 1)
        out["forward_launch_TOPS"] = round(launch_ops / (launch_ms * 1e-3) / 1e12, 2)
        if ceilings:
            if w.m > 16:
                out["forward_frac_of_measured_mfma"] = round(out["forward_launch_TOPS"] / ceilings["mfma_int8_TOPS"], 4)
            else:
                out["forward_frac_of_plain_read"] = round(out["forward_launch_GBps"] / read_ceiling(ceilings,
                                                                                                     launch_bytes), 4)
    return out


# legs that carry their own roofline block: the 2B-class M = 1 decode, the 2048-token
# prefill, and the int8-only decode of the 100B-class matrices
ROOFLINE_LEGS = {"1", "3", "4i"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import bitlinear_fwd_amd as bl
    from bitlinear_fwd_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bl.lib()
    m_head = synth.WORKLOADS[args.workload].m_list[0]
    # the clock and power state before the timed region, read before the workload is built:
    # the tool runs as a child process, and the idle GPU it leaves behind would otherwise
    # slow the first timed steps (measured: 2.062 vs 2.055 ms per headline step)
    state_before = gpu_state()
    head = Workload(bl, synth, args.workload, m_head, dev, path=args.path)
    if args.graph:
        head.capture()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    progress(f"headline workload {args.workload} M={m_head} ready: {len(head.calls[0])} launches per step")
    ms, trials, host_ms = time_steps(head, args.steps, args.warmup)
    state_after = gpu_state()
    progress(f"headline timed: {ms:.4f} ms per step")
    decode = m_head <= 16
    graph = None
    if not args.graph:
        # the same step captured once into a HIP graph and replayed: the launches without the
        # host's issue cost, gaps between the kernels included (reported beside the eager value)
        head.capture()
        g_ms, g_trials, _ = time_steps(head, args.steps, args.warmup)
        head.graphs = None
        graph = {"ms_per_step": round(g_ms, 5), "launch_us": round(g_ms * 1e3 / len(head.calls[0]), 3),
                 "trials": trial_stats(g_trials, head.bytes_per_step(), None if decode else head.ops_per_step())}
        if decode:
            graph["GBps"] = round(head.bytes_per_step() / (g_ms * 1e-3) / 1e9, 1)
        else:
            graph["TOPS"] = round(head.ops_per_step() / (g_ms * 1e-3) / 1e12, 2)
        progress(f"headline as graph replays: {g_ms:.4f} ms per step")
    launch_ms, launch_bytes, launch_ops, launch_timing = launch_timing_of(head, ms)
    value = head.bytes_per_step() / (ms * 1e-3) / 1e9 if decode else head.ops_per_step() / (ms * 1e-3) / 1e12
    ceilings = None if args.skip_ceilings else measure_ceilings(bl, dev)
    progress("ceilings measured")
    roof = roofline_block(head, launch_ms, launch_bytes, launch_ops, launch_timing, args.workload, ceilings)
    quantisers = None if args.skip_ceilings else measure_quantisers(bl, synth, dev)
    legs = {}
    for tok in [t.strip() for t in args.legs.split(",") if t.strip()]:
        flags = tok.lstrip("0123456789")
        idx = int(tok[: len(tok) - len(flags)])
        grouped, subln, gated = "g" in flags, "s" in flags, "f" in flags
        path = "lut" if "l" in flags else ("int8" if "i" in flags else ("binary" if "b" in flags else "fused"))
        if (grouped and idx not in GROUPINGS) or (gated and idx != 1):
            continue
        for m in synth.WORKLOADS[idx].m_list:
            if idx == args.workload and not flags and m == m_head:
                continue  # the headline itself
            plan_of = {"lut": bl.forward_lut_plan, "binary": bl.forward_binary_plan}.get(path)
            if plan_of and any(plan_of(m, n, k) is None for _, k, n in synth.WORKLOADS[idx].matrices):
                continue
            w = Workload(bl, synth, idx, m, dev, subln=subln, path=path, weights_from=head)
            if grouped:
                w.set_grouping(GROUPINGS[idx])
            if gated:
                w.set_gated_pair()
            if args.graph:
                w.capture()
            lms, ltrials, lhost = time_steps(w, leg_steps(w), max(2, -(-100 // len(w.calls[0]))))
            key = f"w{idx}{flags}_m{m}"
            progress(f"leg {key}: {lms:.4f} ms per step")
            if gated or grouped or subln:
                legs[key] = leg_summary(w, lms, ltrials, None, None, None)
                if gated:
                    legs[key]["note"] = ("gate and up in one bitlinear_forward_gated_relu2 launch (squared-ReLU "
                                         "gating epilogue), then down; per-step bytes as the three matrices")
                elif grouped:
                    legs[key]["grouping"] = [[w.wl.matrices[i][0] for i in g] for g in GROUPINGS[idx]]
                    legs[key]["note"] = ("projections of one input in one grouped call (shared activation "
                                         "quantisation); per-step bytes and ops as the ungrouped workload")
                else:
                    legs[key]["kernel"] = dominant_kernel(w)
                    legs[key]["note"] = ("sub-layer RMS normalisation (per-feature gain, eps 1e-5) in front of the "
                                         "quantiser, in the same kernel where the plan fuses it")
                if subln and (gated or grouped):
                    legs[key]["note"] += "; sub-layer RMS normalisation in front of the quantiser"
            else:
                l_ms, l_b, l_o, l_how = launch_timing_of(w, lms)
                legs[key] = leg_summary(w, lms, ltrials, l_ms, l_b, l_o, ceilings)
                legs[key]["kernel"] = {"lut": "k_gemv_lut (table-lookup decode)",
                                       "binary": "k_gemv_bin (1-bit sign-binary decode)"}.get(path) or dominant_kernel(w)
                legs[key]["forward_launch_timing"] = l_how
                if path == "fused":
                    legs[key]["traffic_bytes_per_launch"] = measured_traffic(
                        dominant_kernel(w), idx, m, "fused" if all(w.fused.values()) else "int8")
                else:
                    legs[key]["note"] = ("activation quantiser, then the " +
                                         {"lut": "table-lookup forward (bitlinear_forward_lut)",
                                          "binary": "1-bit sign-binary forward (bitlinear_forward_binary; "
                                                    "packed_GBps counts the 1-bit bytes)"}.get(
                                             path, "int8 forward (bitlinear_forward)") +
                                         "; forward_launch_* time the forward launches alone")
                if tok in ROOFLINE_LEGS and (m == synth.WORKLOADS[idx].m_list[0]):
                    legs[key]["roofline"] = roofline_block(w, l_ms, l_b, l_o, l_how, idx, ceilings)
            legs[key]["host_us_per_launch"] = round(lhost * 1e3 / max(1, len(w.calls[0])), 3)
            if not args.graph and lhost >= 0.9 * lms:
                # the host's issue rate sets this leg's pace: the same step as HIP graph replays,
                # reported beside it (the eager figures above stay the leg's record; measured, graph
                # replay is faster on the one-GPU-shard legs and slower on the short 2B-class ones)
                w.capture()
                g_ms, g_trials, _ = time_steps(w, leg_steps(w), max(2, -(-100 // len(w.calls[0]))))
                w.graphs = None
                legs[key]["graph_replay"] = {
                    "ms_per_step": round(g_ms, 5), "us_per_matrix": round(g_ms * 1e3 / w.matrices_per_step(), 3),
                    "packed_GBps": round(w.bytes_per_step() / (g_ms * 1e-3) / 1e9, 1),
                    "allin_GBps": round(w.allin_bytes_per_step() / (g_ms * 1e-3) / 1e9, 1),
                    "trials": trial_stats(g_trials, w.bytes_per_step(), w.ops_per_step() if w.m > 16 else None)}
                progress(f"leg {key} as graph replays: {g_ms:.4f} ms per step")
            del w
            torch.cuda.empty_cache()
    shapes = time_prefill_shapes(bl, synth, dev, args.prefill_shapes) if args.prefill_shapes else None
    cpu = cpu_single = None
    host = host_cpu_facts()
    if not args.no_cpu_baseline:
        unit = "GB/s" if decode else "TOPS"
        rate = (lambda b, o, t: round(b / t / 1e9, 4)) if decode else (lambda b, o, t: round(o / t / 1e12, 6))
        threads = max(1, min(16, host["physical_cores_in_affinity"]))
        b, o, t, n_done, per_step = cpu_baseline_cores(head, args.cpu_seconds, threads)
        cpu = {"value": rate(b, o, t), "unit": unit, "cores": threads, "kind": "oracle",
               "sample": (f"{n_done} of the step's {per_step} matrices in order "
                          f"({'the whole step' if n_done == per_step else 'a leading sample'}), {t:.1f} s: act quant "
                          f"once per matrix, then each matrix's 16-row blocks split into {threads} contiguous "
                          f"slices (unpack + int matmul + rescale) on {threads} host threads, one per physical "
                          "core of this process's CPU set"),
               "step_s_scaled": round(t * per_step / n_done, 3),
               "tokens_per_s_eq": round(m_head * n_done / (t * per_step), 3),
               "host": host, "oracle_cflags": " ".join(oracle_cflags())}
        progress(f"oracle on {threads} threads: {n_done} matrices in {t:.1f} s")
        b1, o1, t1, n1, per_step = cpu_baseline_single(head, 2)
        progress(f"oracle on one thread: {n1} matrices in {t1:.1f} s")
        scaled = per_step / n1
        cpu_single = {"value": rate(b1, o1, t1), "unit": unit, "cores": 1, "kind": "oracle",
                      "sample": (f"{n1} matrices ({'2 layers' if head.sweep else '2 weight sets'}) on one thread, "
                                 f"{t1:.1f} s; the step time is scaled by {per_step}/{n1} (SCALED, not measured "
                                 "over the whole step)"),
                      "step_s_scaled": round(t1 * scaled, 3),
                      "tokens_per_s_eq_scaled": round(m_head / (t1 * scaled), 4)}
    out = {
        "metric": "BitLinear decode packed-weight GB/s (% HBM peak); prefill int8 TOPS (% MFMA)",
        "value": round(value, 1 if decode else 2),
        "unit": "GB/s" if decode else "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": {"workload": head.wl.name, "M": m_head,
                   "matrices": [list(x) for x in head.wl.matrices],
                   "layers": head.wl.layers, "distinct_weight_sets": len(head.sets),
                   "launches_per_step": len(head.calls[0]),
                   "packed_bytes_per_step": head.bytes_per_step(),
                   "allin_GBps": round(head.allin_bytes_per_step() / (ms * 1e-3) / 1e9, 1),
                   "us_per_matrix": round(ms * 1e3 / head.matrices_per_step(), 3),
                   "tokens_per_s_eq": round(m_head / (ms * 1e-3), 1),
                   "seeds": "torch.Generator per tensor: 1000*workload + 10*layer + matrix for weights, "
                            "+500 for activations, +700 for sub-layer gains",
                   "launch": "hip graph replay" if args.graph else "pre-marshalled eager C-ABI calls",
                   "host_us_per_launch": round(host_ms * 1e3 / max(1, len(head.calls[0])), 3),
                   "path": args.path,
                   "hbm_frac": round(value / HBM_PEAK_GBS, 4) if decode else None},
        "trials": trial_stats(trials, head.bytes_per_step(), None if decode else head.ops_per_step()),
        "graph_replay": graph,
        "roofline": roof,
        "ceilings": ceilings,
        "quantisers": quantisers,
        "cpu_baseline": cpu,
        "cpu_baseline_single_thread": cpu_single,
        "gpu_state": {"before_timed_region": state_before, "after_timed_region": state_after},
        "legs": legs,
        "prefill_shapes": shapes,
    }
    print(json.dumps(out), flush=True)


def progress(msg: str) -> None:
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def oracle_cflags():
    import oracle

    return ["gcc", *oracle._CFLAGS]


if __name__ == "__main__":
    main()
