"""Benchmark of the BitLinear forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload 1] [--legs 2,3,4]
                    [--no-graph] [--no-cpu-baseline] [--copy-calibration MIB]

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

Headline (default workload 1): 2B-class decode at M = 1, gate/up 2560->6912 and down
6912->2560, cycling through 48 distinct weight sets (637 MB of packed weights, more than
twice the 256 MB Infinity Cache) so every step streams its weights from HBM.  value =
packed-weight bytes per step / step time, in GB/s.  The JSON line also carries:
  roofline     the dominant kernel: algorithmic bytes (decode) or int8 ops (prefill) per
               launch / mean launch duration, against 8 TB/s or 5.0 POPS.  The duration
               comes from HIP events on the replay stream: the timed region over its
               launches when the step is nothing but that kernel, else graph replays of the
               forward launches alone.  traffic: measured HBM bytes per launch (see TRAFFIC);
  legs         the other workloads: M = 16 full layer, M = 2048 prefill (int8 TOPS vs
               5.0 POPS dense int8 MFMA), 100B-class M = 1 and M = 8 sweeps, and the 2B
               decode workloads with the projections of one input (gate/up, Q/K/V) grouped
               into one bitlinear_forward_grouped call ("1g", "2g"), and the same
               workloads behind the sub-layer RMS normalisation ("1s", "1gs", "2s"), and the
               gate/up pair with the squared-ReLU gating epilogue in one launch ("1f", "1fs");
               the two-kernel int8 path ("1i"), the table-lookup decode ("1l") and the 1-bit
               sign-binary variant ("1b", "4b") for comparison with the ternary decode, and
               one GPU's share of the 100B-class matrices split over 8 GPUs ("5": the up
               projection's 3584 output rows, the down projection's 3584 input columns);
  gpu_state    rocm-smi clock and power readings before and after the timed region;
  quantisers   the weight quantiser (2560 -> 6912 fp32 latents) and the activation quantiser
               (bf16, decode and prefill sizes) timed alone, in bytes moved per second;
  ceilings     measured on this GPU by the library's probes: HBM read rate with the decode
               access pattern at 58.7 MB and 4.4 MB per launch, and the int8 MFMA rate;
               roofline.frac_of_measured_ceiling sets the dominant kernel against the
               one that matches its size;
  cpu_baseline the CPU oracle on the host, on a bounded sample of the same workload.
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
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3, 4, 5])
    ap.add_argument("--legs", default="1g,1s,1gs,1f,1fs,1i,1l,1b,2,2g,2s,3,4,4b,5",
                    help="other workloads timed into 'legs' ('' for none); a trailing g times the workload "
                         "with the projections of one input grouped into one call")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph instead of pre-marshalled eager launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device three times (the reference kernel of "
                         "known size for scaling FETCH_SIZE / WRITE_SIZE counter runs)")
    return ap.parse_args()


class Matrix:
    """One quantised weight matrix with its pre-drawn activations."""

    def __init__(self, bl, synth, wl, layer, midx, k, n, m, dev, binary=False):
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
    def __init__(self, bl, synth, idx, m, dev, subln=False, path="fused"):
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
        self.sets = [[Matrix(bl, synth, self.wl, s, i, k, n, m, dev, binary=path == "binary")
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
        import torch

        self.graphs = []
        for group in self.step_groups():
            for mat in group:  # warm the kernels once outside capture
                self.launch(mat)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for mat in group:
                    self.launch(mat)
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
    # (workload, M): scaled bytes per launch (fetch + write), raw KiB per launch, source hash.
    # Copy calibration (256 MiB device copy): FETCH_SIZE read 131085.3 KiB (x1.99980),
    # WRITE_SIZE 262144.0 KiB (x1.0).
    (1, 1): {"bytes_per_launch": 4591108, "fetch_kib": 2229.34, "write_kib": 25.28, "sha": "61f7a96371860d6d"},
    (2, 16): {"bytes_per_launch": 3160075, "fetch_kib": 1441.44, "write_kib": 203.43, "sha": "61f7a96371860d6d"},
    (3, 2048): {"bytes_per_launch": 94794700, "fetch_kib": 27345.22, "write_kib": 37888.06, "sha": "85d7b679bf307030"},
    (4, 1): {"bytes_per_launch": 59258200, "fetch_kib": 28892.26, "write_kib": 90.03, "sha": "61f7a96371860d6d"},
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


def measured_traffic(kernel: str, workload: int, m: int):
    rec = TRAFFIC.get((workload, m))
    if rec is None:
        return None
    kind = "prefill" if kernel.startswith("k_gemm") else "decode"
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


def measure_ceilings(bl, dev):
    """Measured ceilings on this GPU (library probes, back-to-back launches timed with HIP
    events): HBM read rate for the decode access pattern at the two matrix sizes (the
    buffers rotate through 2 GiB, so every launch reads from HBM), and the int8 MFMA rate
    with no memory traffic."""
    import torch

    pool_bytes = 2 << 30
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    pool.fill_(0x5A)
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, nbytes in (("58.7MB", 58_720_256), ("4.4MB", 4_423_680)):
        copies = pool_bytes // nbytes
        words = int(bl.lib().bitlinear_probe_stream_words(nbytes))
        sink = torch.empty(words, dtype=torch.int32, device=dev)
        calls = [bl.PreparedCall("bitlinear_probe_stream", pool.data_ptr() + i * nbytes, nbytes, sink.data_ptr(),
                                 words, stream) for i in range(copies)]
        reps = 400 if nbytes < 10_000_000 else 200
        for i in range(20):
            calls[i % copies]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            calls[i % copies]()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[f"stream_{name}_us"] = round(us, 3)
        out[f"stream_{name}_GBps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    del pool
    torch.cuda.empty_cache()
    # about 5 ms per launch; the first launch brings the clocks up, the best of three counts
    groups, iters = 512, 16000
    sink = torch.empty(groups, dtype=torch.int32, device=dev)
    best = 0.0
    for rep in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bl.probe_mfma(iters, groups, sink)
        e1.record()
        torch.cuda.synchronize()
        if rep:
            best = max(best, 2.0 * 16 * 16 * 64 * 16 * iters * groups * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    out["mfma_int8_TOPS"] = round(best, 1)
    return out


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
    import torch

    for _ in range(warmup):
        w.run_step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        w.run_step()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per step


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


def cpu_baseline(w: Workload, budget_s: float):
    """The oracle on the host over a bounded sample of the same workload (one thread)."""
    import numpy as np
    import torch

    import oracle

    def acts_host_f32(x):
        if x.dtype == torch.bfloat16:
            return oracle.bf16_bits_to_f32(x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        return x.float().cpu().numpy()

    done_bytes, done_ops, t_used, mats = 0, 0, 0.0, 0
    for mat in sum(w.sets, []):
        packed = mat.packed.cpu().numpy()
        x = acts_host_f32(mat.x)
        g = np.float32(mat.gamma.cpu().numpy()[0])
        t0 = time.perf_counter()
        xq, a = oracle.quant_acts(x)
        q = oracle.unpack(packed, mat.n, mat.k)
        oracle.forward(q, g, xq, a, mat.k)
        t_used += time.perf_counter() - t0
        done_bytes += mat.bytes
        done_ops += mat.ops
        mats += 1
        if t_used >= budget_s:
            break
    return done_bytes, done_ops, t_used, mats


def cpu_baseline_threads(w: Workload, budget_s: float, threads: int):
    """The same oracle calls on `threads` host threads at once (the oracle's C routines run
    outside the interpreter lock), each thread taking whole matrices of the workload in
    turn until the wall-clock budget is spent: the oracle as it is, on more cores."""
    import threading

    import numpy as np
    import torch

    import oracle

    def acts_host_f32(x):
        if x.dtype == torch.bfloat16:
            return oracle.bf16_bits_to_f32(x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        return x.float().cpu().numpy()

    mats = sum(w.sets, [])[: 4 * threads]
    inputs = [(m.packed.cpu().numpy(), acts_host_f32(m.x), np.float32(m.gamma.cpu().numpy()[0]), m) for m in mats]
    lock = threading.Lock()
    state = {"next": 0, "bytes": 0, "ops": 0, "mats": 0}
    t0 = time.perf_counter()

    def worker():
        while time.perf_counter() - t0 < budget_s:
            with lock:
                i = state["next"]
                state["next"] += 1
            packed, x, g, mat = inputs[i % len(inputs)]
            xq, a = oracle.quant_acts(x)
            q = oracle.unpack(packed, mat.n, mat.k)
            oracle.forward(q, g, xq, a, mat.k)
            with lock:
                state["bytes"] += mat.bytes
                state["ops"] += mat.ops
                state["mats"] += 1

    pool = [threading.Thread(target=worker) for _ in range(threads)]
    for t in pool:
        t.start()
    for t in pool:
        t.join()
    return state["bytes"], state["ops"], time.perf_counter() - t0, state["mats"]


def leg_summary(w: Workload, ms: float, launch_ms, launch_bytes, launch_ops, ceilings=None):
    gbs = w.bytes_per_step() / (ms * 1e-3) / 1e9
    tops = w.ops_per_step() / (ms * 1e-3) / 1e12
    out = {
        "workload": w.wl.name, "M": w.m, "ms_per_step": round(ms, 5),
        "us_per_matrix": round(ms * 1e3 / w.matrices_per_step(), 3),
        "packed_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "allin_GBps": round(w.allin_bytes_per_step() / (ms * 1e-3) / 1e9, 1),
        "int8_TOPS": round(tops, 2), "mfma_frac": round(tops / I8_PEAK_TOPS, 4),
        "tokens_per_s_eq": round(w.m / (ms * 1e-3), 1),  # every matrix of the step applied once per token
    }
    if launch_ms is not None:
        out["forward_launch_us"] = round(launch_ms * 1e3, 3)
        out["forward_launch_GBps"] = round(launch_bytes / (launch_ms * 1e-3) / 1e9, 1)
        out["forward_launch_TOPS"] = round(launch_ops / (launch_ms * 1e-3) / 1e12, 2)
        if ceilings:
            if w.m > 16:
                out["forward_frac_of_measured_mfma"] = round(out["forward_launch_TOPS"] / ceilings["mfma_int8_TOPS"], 4)
            else:
                big = launch_bytes >= 20e6
                c = ceilings["stream_58.7MB_GBps"] if big else ceilings["stream_4.4MB_GBps"]
                out["forward_frac_of_measured_stream"] = round(out["forward_launch_GBps"] / c, 4)
    return out


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
    head = Workload(bl, synth, args.workload, m_head, dev)
    if args.graph:
        head.capture()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    state_before = gpu_state()
    ms = time_steps(head, args.steps, args.warmup)
    state_after = gpu_state()
    decode = m_head <= 16
    mats = head.step_groups()[0]
    if all(head.fused.values()):
        # the step holds nothing but launches of the fused kernel: its mean launch duration
        # is the timed region (HIP events on the replay stream) over the launches in it
        launch_ms = ms / len(mats)
        launch_bytes, launch_ops = head.bytes_per_step() / len(mats), head.ops_per_step() / len(mats)
        launch_timing = "timed region / launches (the step is only this kernel)"
    else:
        launch_ms, launch_bytes, launch_ops = time_forward_only(head, 3 if head.sweep else max(40, 4 * len(head.sets)))
        launch_timing = "graph replays of the forward launches alone"
    value = head.bytes_per_step() / (ms * 1e-3) / 1e9 if decode else head.ops_per_step() / (ms * 1e-3) / 1e12
    kernel = dominant_kernel(head)
    traffic = measured_traffic(kernel, args.workload, m_head)
    if decode:
        achieved = launch_bytes / (launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kernel, "launch_us": round(launch_ms * 1e3, 3), "launch_timing": launch_timing,
                "algorithmic_bytes_per_launch": int(launch_bytes)}
    else:
        # int8 contraction: TOPS against the dense int8 MFMA peak (unit kept as the contract's)
        achieved = launch_ops / (launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": I8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(achieved / I8_PEAK_TOPS, 4), "traffic": traffic, "kernel": kernel,
                "launch_us": round(launch_ms * 1e3, 3), "launch_timing": launch_timing,
                "algorithmic_ops_per_launch": int(launch_ops)}
    ceilings = measure_ceilings(bl, dev)
    quantisers = measure_quantisers(bl, synth, dev)
    if decode:
        ceil = ceilings["stream_4.4MB_GBps"] if head.bytes_per_step() / len(mats) < 20e6 else ceilings["stream_58.7MB_GBps"]
    else:
        ceil = ceilings["mfma_int8_TOPS"]
    roof["measured_ceiling"] = ceil
    roof["frac_of_measured_ceiling"] = round(roof["achieved"] / ceil, 4)
    if decode:
        roof["note"] = ("algorithmic bytes are the 2-bit packed weights; the information bound of ternary "
                        "codes, log2(3) bits per weight, is 79 % of them")
    legs = {}
    for tok in [t.strip() for t in args.legs.split(",") if t.strip()]:
        flags = tok.lstrip("0123456789")
        idx = int(tok[: len(tok) - len(flags)])
        grouped, subln, gated = "g" in flags, "s" in flags, "f" in flags
        path = "lut" if "l" in flags else ("int8" if "i" in flags else ("binary" if "b" in flags else "fused"))
        if idx == args.workload and not flags:
            continue
        if (grouped and idx not in GROUPINGS) or (gated and idx != 1):
            continue
        for m in synth.WORKLOADS[idx].m_list:
            plan_of = {"lut": bl.forward_lut_plan, "binary": bl.forward_binary_plan}.get(path)
            if plan_of and any(plan_of(m, n, k) is None for _, k, n in synth.WORKLOADS[idx].matrices):
                continue
            w = Workload(bl, synth, idx, m, dev, subln=subln, path=path)
            if grouped:
                w.set_grouping(GROUPINGS[idx])
            if gated:
                w.set_gated_pair()
            if args.graph:
                w.capture()
            steps = max(3, args.steps // (40 if w.sweep else 1))
            lms = time_steps(w, steps, max(1, args.warmup // (40 if w.sweep else 4)))
            key = f"w{idx}{flags}_m{m}"
            if gated:
                legs[key] = leg_summary(w, lms, None, None, None)
                legs[key]["note"] = ("gate and up in one bitlinear_forward_gated_relu2 launch (squared-ReLU gating "
                                     "epilogue), then down; per-step bytes as the three matrices")
                if subln:
                    legs[key]["note"] += "; sub-layer RMS normalisation in front of both quantisers"
            elif grouped:
                legs[key] = leg_summary(w, lms, None, None, None)
                legs[key]["grouping"] = [[w.wl.matrices[i][0] for i in g] for g in GROUPINGS[idx]]
                legs[key]["note"] = ("projections of one input in one grouped call (shared activation "
                                     "quantisation); per-step bytes and ops as the ungrouped workload")
                if subln:
                    legs[key]["note"] += "; sub-layer RMS normalisation in front of the quantiser"
            elif path != "fused":
                l_ms, l_b, l_o = time_forward_only(w, 3 if w.sweep else max(40, 4 * len(w.sets)))
                legs[key] = leg_summary(w, lms, l_ms, l_b, l_o, ceilings)
                legs[key]["kernel"] = {"lut": "k_gemv_lut (table-lookup decode)",
                                       "binary": "k_gemv_bin (1-bit sign-binary decode)"}.get(path) or dominant_kernel(w)
                legs[key]["note"] = ("activation quantiser, then the " +
                                     {"lut": "table-lookup forward (bitlinear_forward_lut)",
                                      "binary": "1-bit sign-binary forward (bitlinear_forward_binary; "
                                                "packed_GBps counts the 1-bit bytes)"}.get(
                                         path, "int8 forward (bitlinear_forward)") +
                                     "; forward_launch_* time the forward launches alone")
            elif subln:
                legs[key] = leg_summary(w, lms, None, None, None)
                legs[key]["kernel"] = dominant_kernel(w)
                legs[key]["note"] = ("sub-layer RMS normalisation (per-feature gain, eps 1e-5) in front of the "
                                     "quantiser, in the same kernel where the plan fuses it")
            else:
                l_ms, l_b, l_o = time_forward_only(w, 3 if w.sweep else max(40, 4 * len(w.sets)))
                legs[key] = leg_summary(w, lms, l_ms, l_b, l_o, ceilings)
                legs[key]["kernel"] = dominant_kernel(w)
                legs[key]["traffic_bytes_per_launch"] = measured_traffic(dominant_kernel(w), idx, m)
            del w
            torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        b, o, t, n_cpu = cpu_baseline(head, args.cpu_seconds)
        threads = min(16, len(os.sched_getaffinity(0)))
        bm, om, tm, nm = cpu_baseline_threads(head, args.cpu_seconds / 2, threads)
        cpu_mt = {"value": round(bm / tm / 1e9, 4) if decode else round(om / tm / 1e12, 6),
                  "unit": "GB/s" if decode else "TOPS", "cores": threads, "kind": "oracle",
                  "sample": f"{nm} matrices of the same workload on {threads} host threads at once, "
                            f"{tm:.1f} s wall clock"}
        cpu = {"value": round(b / t / 1e9, 4) if decode else round(o / t / 1e12, 6),
               "unit": "GB/s" if decode else "TOPS", "cores": 1, "kind": "oracle",
               "sample": f"{n_cpu} matrices of the same workload (act quant + unpack + int matmul + rescale), "
                         f"{t:.1f} s, single-threaded scalar C"}
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
                   "distinct_weight_sets": len(head.sets),
                   "packed_bytes_per_step": head.bytes_per_step(),
                   "allin_GBps": round(head.allin_bytes_per_step() / (ms * 1e-3) / 1e9, 1),
                   "us_per_matrix": round(ms * 1e3 / head.matrices_per_step(), 3),
                   "tokens_per_s_eq": round(m_head / (ms * 1e-3), 1),
                   "seeds": "torch.Generator per tensor: 1000*workload + 10*set + matrix for weights, "
                            "+500 for activations, +700 for sub-layer gains",
                   "launch": "hip graph replay" if args.graph else "pre-marshalled eager C-ABI calls",
                   "hbm_frac": round(value / HBM_PEAK_GBS, 4) if decode else None},
        "roofline": roof,
        "ceilings": ceilings,
        "quantisers": quantisers,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_mt if cpu else None,
        "gpu_state": {"before_timed_region": state_before, "after_timed_region": state_after},
        "legs": legs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
