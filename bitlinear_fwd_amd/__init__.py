"""MI355X-native BitNet b1.58 BitLinear forward: thin Python binding of libbitlinear.so.

The binding only marshals arguments: every step of the path (weight absmean + ternarise
+ pack, per-token absmax int8 activation quantisation, the packed-ternary x int8
contraction with exact int32 accumulation, and the fp32 rescale) runs in the HIP kernels
behind the C ABI declared in ``include/bitlinear.h``.  PyTorch supplies device memory
and the current stream.  There is no CPU fallback: if the library is missing or a call
fails, an exception is raised.

The method follows the aratech.ae article "BitNet b1.58: Microsoft's 1-bit LLM that runs
a 100B model on one CPU" (sub-sections "Ternary weights {-1, 0, +1}" and "BitLinear: the
building block") and the 2-bit code table of bhfrc.com news 56965, section 4.1.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

BL_OK, BL_ERR_INVALID_ARG, BL_ERR_UNSUPPORTED, BL_ERR_HIP = 0, -1, -2, -3
BL_F32, BL_BF16 = 0, 1

_lib = None


class BitLinearError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libbitlinear.so (built by ``python -m bitlinear_fwd_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bitlinear_fwd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, p, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.bitlinear_version.restype = c_int
        L.bitlinear_version.argtypes = []
        L.bitlinear_status_string.restype = ctypes.c_char_p
        L.bitlinear_status_string.argtypes = [c_int]
        for name in ("bitlinear_n_pad", "bitlinear_k_pad"):
            getattr(L, name).restype = i64
            getattr(L, name).argtypes = [i64]
        for name in ("bitlinear_packed_bytes", "bitlinear_wq_workspace_bytes"):
            getattr(L, name).restype = i64
            getattr(L, name).argtypes = [i64, i64]
        L.bitlinear_quantize_weights.restype = c_int
        L.bitlinear_quantize_weights.argtypes = [p, i64, i64, p, p, p, i64, p]
        L.bitlinear_quantize_weights_noalloc.restype = c_int
        L.bitlinear_quantize_weights_noalloc.argtypes = [p, i64, i64, p, p, p]
        L.bitlinear_quantize_acts.restype = c_int
        L.bitlinear_quantize_acts.argtypes = [p, c_int, i64, i64, p, p, p, p]
        L.bitlinear_forward_fused.restype = c_int
        L.bitlinear_forward_fused.argtypes = [p, p, p, c_int, i64, i64, i64, p, p, p, p, p]
        L.bitlinear_forward_plan.restype = c_int
        L.bitlinear_forward_plan.argtypes = [i64, i64, i64, p]
        L.bitlinear_forward_fused_plan.restype = c_int
        L.bitlinear_forward_fused_plan.argtypes = [i64, i64, i64, c_int, p]
        L.bitlinear_forward.restype = c_int
        L.bitlinear_forward.argtypes = [p, p, p, p, i64, i64, i64, p, p, p]
        L.bitlinear_forward_ws_bytes.restype = i64
        L.bitlinear_forward_ws_bytes.argtypes = [i64, i64, i64]
        L.bitlinear_forward_ws.restype = c_int
        L.bitlinear_forward_ws.argtypes = [p, p, p, p, i64, i64, i64, p, p, p, i64, p]
        L.bitlinear_probe_prefill_occupancy.restype = c_int
        L.bitlinear_probe_prefill_occupancy.argtypes = [p]
        L.bitlinear_forward_ws_plan.restype = c_int
        L.bitlinear_forward_ws_plan.argtypes = [i64, i64, i64, p]
        L.bitlinear_probe_stream_words.restype = i64
        L.bitlinear_probe_stream_words.argtypes = [i64]
        L.bitlinear_probe_stream.restype = c_int
        L.bitlinear_probe_stream.argtypes = [p, i64, p, i64, p]
        L.bitlinear_probe_read.restype = c_int
        L.bitlinear_probe_read.argtypes = [p, i64, i64, c_int, p, p]
        L.bitlinear_probe_mfma.restype = c_int
        L.bitlinear_probe_mfma.argtypes = [i64, i64, p, p]
        L.bitlinear_forward_grouped.restype = c_int
        L.bitlinear_forward_grouped.argtypes = [p, c_int, p, c_int, i64, i64, p, p, p]
        f32 = ctypes.c_float
        L.bitlinear_subln_quantize_acts.restype = c_int
        L.bitlinear_subln_quantize_acts.argtypes = [p, c_int, i64, i64, p, f32, p, p, p]
        L.bitlinear_forward_subln.restype = c_int
        L.bitlinear_forward_subln.argtypes = [p, p, p, c_int, i64, i64, i64, p, f32, p, p, p, p, p]
        L.bitlinear_forward_grouped_subln.restype = c_int
        L.bitlinear_forward_grouped_subln.argtypes = [p, c_int, p, c_int, i64, i64, p, f32, p, p, p]
        L.bitlinear_gated_relu2_workspace_bytes.restype = i64
        L.bitlinear_gated_relu2_workspace_bytes.argtypes = [i64, i64]
        L.bitlinear_forward_gated_relu2.restype = c_int
        L.bitlinear_forward_gated_relu2.argtypes = [p, p, p, p, p, c_int, i64, i64, i64, c_int, p, f32, p, p, p, p,
                                                    i64, p]
        L.bitlinear_forward_gated_relu2_plan.restype = c_int
        L.bitlinear_forward_gated_relu2_plan.argtypes = [i64, i64, i64, c_int, c_int, p]
        for name in ("bitlinear_kb_pad",):
            getattr(L, name).restype = i64
            getattr(L, name).argtypes = [i64]
        L.bitlinear_packed_bytes_binary.restype = i64
        L.bitlinear_packed_bytes_binary.argtypes = [i64, i64]
        L.bitlinear_quantize_weights_binary.restype = c_int
        L.bitlinear_quantize_weights_binary.argtypes = [p, i64, i64, p, p, p, i64, p]
        L.bitlinear_forward_binary.restype = c_int
        L.bitlinear_forward_binary.argtypes = [p, p, p, p, i64, i64, i64, p, p, p]
        L.bitlinear_forward_binary_plan.restype = c_int
        L.bitlinear_forward_binary_plan.argtypes = [i64, i64, i64, p]
        L.bitlinear_forward_lut.restype = c_int
        L.bitlinear_forward_lut.argtypes = [p, p, p, p, i64, i64, i64, p, p, p]
        L.bitlinear_forward_lut_plan.restype = c_int
        L.bitlinear_forward_lut_plan.argtypes = [i64, i64, i64, p]
        L.bitlinear_forward_subln_plan.restype = c_int
        L.bitlinear_forward_subln_plan.argtypes = [i64, i64, i64, c_int, p]
        _lib = L
    return _lib


EXPORTED_SYMBOLS = (
    "bitlinear_version", "bitlinear_status_string", "bitlinear_n_pad", "bitlinear_k_pad",
    "bitlinear_packed_bytes", "bitlinear_wq_workspace_bytes", "bitlinear_quantize_weights",
    "bitlinear_quantize_acts", "bitlinear_forward", "bitlinear_forward_fused", "bitlinear_forward_plan",
    "bitlinear_forward_fused_plan", "bitlinear_forward_grouped", "bitlinear_probe_stream_words",
    "bitlinear_probe_stream", "bitlinear_probe_read", "bitlinear_probe_mfma", "bitlinear_subln_quantize_acts",
    "bitlinear_forward_subln",
    "bitlinear_forward_grouped_subln", "bitlinear_forward_subln_plan", "bitlinear_gated_relu2_workspace_bytes",
    "bitlinear_forward_gated_relu2", "bitlinear_forward_gated_relu2_plan", "bitlinear_forward_lut",
    "bitlinear_forward_lut_plan", "bitlinear_kb_pad", "bitlinear_packed_bytes_binary",
    "bitlinear_quantize_weights_binary", "bitlinear_forward_binary", "bitlinear_forward_binary_plan",
    "bitlinear_quantize_weights_noalloc", "bitlinear_forward_ws_bytes", "bitlinear_forward_ws",
    "bitlinear_forward_ws_plan", "bitlinear_probe_prefill_occupancy",
)

MAX_GROUP = 8


class BlMatrix(ctypes.Structure):
    """bl_matrix of bitlinear.h: one weight matrix of a grouped call."""
    _fields_ = [("packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("Y", ctypes.c_void_p), ("acc", ctypes.c_void_p)]


def _check(fn: str, status: int) -> None:
    if status != BL_OK:
        raise BitLinearError(fn, status, lib().bitlinear_status_string(status).decode())


def status_string(status: int) -> str:
    return lib().bitlinear_status_string(status).decode()


def version() -> int:
    return lib().bitlinear_version()


def n_pad(n: int) -> int:
    return int(lib().bitlinear_n_pad(n))


def k_pad(k: int) -> int:
    return int(lib().bitlinear_k_pad(k))


def packed_bytes(n: int, k: int) -> int:
    return int(lib().bitlinear_packed_bytes(n, k))


def wq_workspace_bytes(n: int, k: int) -> int:
    return int(lib().bitlinear_wq_workspace_bytes(n, k))


def _plan_dict(out) -> dict:
    if out[0] == 5:
        return {"kernel": "binary", "workgroups": out[1], "threads": out[2], "row_blocks": out[3],
                "tiles_per_wave": out[4]}
    if out[0] == 4:
        return {"kernel": "lut", "workgroups": out[1], "threads": out[2], "row_blocks": out[3],
                "tiles_per_wave": out[4], "lds_bytes": out[5]}
    if out[0] == 3 and out[4] == 4:  # 5..16 tokens: every workgroup quantises the 16 token rows into LDS
        return {"kernel": "fused", "workgroups": out[1], "threads": out[2], "row_blocks": out[3],
                "acts": "lds16", "lds_acts": True, "lds_bytes": 0, "tiles_per_wave": out[5]}
    if out[0] == 3:
        return {"kernel": "fused", "workgroups": out[1], "threads": out[2], "row_blocks": out[3],
                "acts": "registers" if out[4] == 2 else "lds", "lds_acts": out[4] == 1,
                "lds_bytes": out[5] if out[4] == 1 else 0, "tiles_per_wave": out[5] if out[4] == 2 else 0}
    if out[0] == 1:
        acts = {0: "per-tile loads", 1: "lds", 2: "registers"}[out[4]]
        return {"kernel": "decode", "workgroups": out[1], "threads": out[2], "row_blocks": out[3],
                "acts": acts, "lds_acts": out[4] == 1, "lds_bytes": out[5] if out[4] == 1 else 0,
                "tiles_per_wave": out[5] if out[4] == 2 else 0}
    d = {"kernel": "prefill", "workgroups": out[1], "threads": out[2], "tile_m": out[3], "tile_n": out[4],
         "k_groups": out[5]}
    if out[0] == 6:
        d.update(split_tail=True, rounds=out[6], split_tiles=out[7], k_ranges=out[8], chunks_per_range=out[9])
    return d


def forward_plan(m: int, n: int, k: int) -> dict:
    """The launch bitlinear_forward makes for (M, N, K), computed on the host."""
    out = (ctypes.c_int32 * 6)()
    _check("bitlinear_forward_plan", lib().bitlinear_forward_plan(m, n, k, out))
    return _plan_dict(out)


def forward_ws_plan(m: int, n: int, k: int) -> dict:
    """The launch bitlinear_forward_ws makes for (M, N, K), computed on the host."""
    out = (ctypes.c_int32 * 10)()
    _check("bitlinear_forward_ws_plan", lib().bitlinear_forward_ws_plan(m, n, k, out))
    return _plan_dict(out)


def forward_ws_bytes(m: int, n: int, k: int) -> int:
    """Workspace bytes bitlinear_forward_ws needs for (M, N, K) (0: none)."""
    v = int(lib().bitlinear_forward_ws_bytes(m, n, k))
    if v < 0:
        raise ValueError(f"invalid shape {(m, n, k)}")
    return v


def forward_workspace(m: int, n: int, k: int, device):
    """A workspace for bitlinear_forward_ws on (M, N, K) (None when it needs none).  Its
    contents on entry do not matter and nothing carries over between calls, so one
    workspace serves later calls of any shape it is large enough for."""
    import torch

    nb = forward_ws_bytes(m, n, k)
    return torch.zeros(nb, dtype=torch.uint8, device=device) if nb > 0 else None


def forward_fused_plan(m: int, n: int, k: int, dtype: str = "bf16") -> dict:
    """What bitlinear_forward_fused does for (M, N, K): kernel "fused" (one launch) or the
    forward launch that follows the activation quantiser."""
    out = (ctypes.c_int32 * 6)()
    dt = BL_BF16 if dtype == "bf16" else BL_F32
    _check("bitlinear_forward_fused_plan", lib().bitlinear_forward_fused_plan(m, n, k, dt, out))
    return _plan_dict(out)


def forward_subln_plan(m: int, n: int, k: int, dtype: str = "bf16") -> dict:
    """What bitlinear_forward_subln does for (M, N, K): kernel "fused" (one launch) or the
    forward launch that follows the normalising quantiser."""
    out = (ctypes.c_int32 * 6)()
    dt = BL_BF16 if dtype == "bf16" else BL_F32
    _check("bitlinear_forward_subln_plan", lib().bitlinear_forward_subln_plan(m, n, k, dt, out))
    return _plan_dict(out)


def forward_gated_relu2_plan(m: int, n: int, k: int, dtype: str = "bf16", subln: bool = False) -> dict:
    """What bitlinear_forward_gated_relu2 does for (M, N, K): kernel "fused" (one launch)
    or the plan of each of the two forwards."""
    out = (ctypes.c_int32 * 6)()
    dt = BL_BF16 if dtype == "bf16" else BL_F32
    _check("bitlinear_forward_gated_relu2_plan",
           lib().bitlinear_forward_gated_relu2_plan(m, n, k, dt, int(subln), out))
    return _plan_dict(out)


def _stream(device) -> int:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def _require_cuda(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize_weights(W, packed=None, gamma=None, workspace=None):
    """Ternarise + pack latent weights W[N][K] (fp32, out x in) on the GPU.

    Returns ``(packed uint8 [packed_bytes(N, K)], gamma fp32 [1])``."""
    import torch

    _require_cuda(W, "W")
    if W.dtype != torch.float32 or W.dim() != 2:
        raise ValueError("W must be a 2-D float32 tensor")
    n, k = W.shape
    dev = W.device
    if packed is None:
        packed = torch.empty(packed_bytes(n, k), dtype=torch.uint8, device=dev)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(wq_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
    _check("bitlinear_quantize_weights", lib().bitlinear_quantize_weights(
        W.data_ptr(), n, k, packed.data_ptr(), gamma.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(dev)))
    return packed, gamma


def quantize_weights_noalloc(W, packed=None, gamma=None):
    """bitlinear_quantize_weights_noalloc: the weight quantiser with the library's own static
    scratch in place of a workspace (the C call allocates nothing; outputs not given here
    are allocated by torch before it).  Returns ``(packed, gamma)``."""
    import torch

    _require_cuda(W, "W")
    if W.dtype != torch.float32 or W.dim() != 2:
        raise ValueError("W must be a 2-D float32 tensor")
    n, k = W.shape
    dev = W.device
    if packed is None:
        packed = torch.empty(packed_bytes(n, k), dtype=torch.uint8, device=dev)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=dev)
    _check("bitlinear_quantize_weights_noalloc", lib().bitlinear_quantize_weights_noalloc(
        W.data_ptr(), n, k, packed.data_ptr(), gamma.data_ptr(), _stream(dev)))
    return packed, gamma


def quantize_acts(x, xq=None, absmax=None, rowsum=None, want_rowsum: bool = False):
    """Per-token absmax int8 quantisation of x[M][K] (fp32 or bf16) on the GPU.

    Returns ``(xq int8 [M][K_pad], absmax fp32 [M])``, plus the exact int32 row sums of
    the codes when ``want_rowsum`` is set or ``rowsum`` is given."""
    import torch

    _require_cuda(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [tokens, features]")
    if x.dtype == torch.float32:
        dt = BL_F32
    elif x.dtype == torch.bfloat16:
        dt = BL_BF16
    else:
        raise ValueError("x must be float32 or bfloat16")
    m, k = x.shape
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k_pad(k)), dtype=torch.int8, device=dev)
    if absmax is None:
        absmax = torch.empty(m, dtype=torch.float32, device=dev)
    if want_rowsum and rowsum is None:
        rowsum = torch.empty(m, dtype=torch.int32, device=dev)
    _check("bitlinear_quantize_acts", lib().bitlinear_quantize_acts(
        x.data_ptr(), dt, m, k, xq.data_ptr(), absmax.data_ptr(), rowsum.data_ptr() if rowsum is not None else None,
        _stream(dev)))
    return (xq, absmax, rowsum) if rowsum is not None else (xq, absmax)


def forward(packed, gamma, xq, absmax, n: int, k: int, y=None, acc=None, want_y: bool = True,
            want_acc: bool = False):
    """y[M][N] (fp32) and/or acc[M][N] (int32) of the packed-ternary x int8 product.

    Returns y, acc or (y, acc) depending on ``want_y`` / ``want_acc``."""
    import torch

    for t, name in ((packed, "packed"), (gamma, "gamma"), (xq, "xq"), (absmax, "absmax")):
        _require_cuda(t, name)
    m = xq.shape[0]
    dev = xq.device
    if want_y and y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    _check("bitlinear_forward", lib().bitlinear_forward(
        packed.data_ptr(), gamma.data_ptr(), xq.data_ptr(), absmax.data_ptr(), m, n, k,
        y.data_ptr() if y is not None else None, acc.data_ptr() if acc is not None else None,
        _stream(dev)))
    if want_y and want_acc:
        return y, acc
    return y if want_y else acc


def forward_ws(packed, gamma, xq, absmax, n: int, k: int, workspace=None, y=None, acc=None, want_y: bool = True,
               want_acc: bool = False):
    """forward() through bitlinear_forward_ws: the same results, with the caller's
    zero-filled workspace (forward_workspace) for the prefill GEMM's split tail tiles."""
    import torch

    for t, name in ((packed, "packed"), (gamma, "gamma"), (xq, "xq"), (absmax, "absmax")):
        _require_cuda(t, name)
    m = xq.shape[0]
    dev = xq.device
    if workspace is not None:
        _require_cuda(workspace, "workspace")
    if want_y and y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    _check("bitlinear_forward_ws", lib().bitlinear_forward_ws(
        packed.data_ptr(), gamma.data_ptr(), xq.data_ptr(), absmax.data_ptr(), m, n, k,
        y.data_ptr() if y is not None else None, acc.data_ptr() if acc is not None else None,
        workspace.data_ptr() if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(dev)))
    if want_y and want_acc:
        return y, acc
    return y if want_y else acc


def kb_pad(k: int) -> int:
    return int(lib().bitlinear_kb_pad(k))


def packed_bytes_binary(n: int, k: int) -> int:
    return int(lib().bitlinear_packed_bytes_binary(n, k))


def quantize_weights_binary(W, packed=None, beta=None, workspace=None):
    """1-bit sign-binary weights: (packed binary buffer, beta = exact mean |W|) on the GPU."""
    import torch

    _require_cuda(W, "W")
    if W.dtype != torch.float32 or W.dim() != 2:
        raise ValueError("W must be a 2-D float32 tensor")
    W = W.contiguous()
    n, k = W.shape
    dev = W.device
    if packed is None:
        packed = torch.empty(packed_bytes_binary(n, k), dtype=torch.uint8, device=dev)
    if beta is None:
        beta = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(wq_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
    _check("bitlinear_quantize_weights_binary", lib().bitlinear_quantize_weights_binary(
        W.data_ptr(), n, k, packed.data_ptr(), beta.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(dev)))
    return packed, beta


def forward_binary_plan(m: int, n: int, k: int):
    """The launch bitlinear_forward_binary makes for (M, N, K), or None where it does not apply."""
    out = (ctypes.c_int32 * 6)()
    st = lib().bitlinear_forward_binary_plan(m, n, k, out)
    if st == BL_ERR_UNSUPPORTED:
        return None
    _check("bitlinear_forward_binary_plan", st)
    return _plan_dict(out)


def forward_binary(packed, beta, xq, absmax, n: int, k: int, y=None, acc=None, want_y: bool = True,
                   want_acc: bool = False):
    """bitlinear_forward with 1-bit sign-binary weights (M <= 4)."""
    import torch

    for t, name in ((packed, "packed"), (beta, "beta"), (xq, "xq"), (absmax, "absmax")):
        _require_cuda(t, name)
    m = xq.shape[0]
    dev = xq.device
    if want_y and y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    _check("bitlinear_forward_binary", lib().bitlinear_forward_binary(
        packed.data_ptr(), beta.data_ptr(), xq.data_ptr(), absmax.data_ptr(), m, n, k,
        y.data_ptr() if y is not None else None, acc.data_ptr() if acc is not None else None, _stream(dev)))
    if want_y and want_acc:
        return y, acc
    return y if want_y else acc


def forward_lut_plan(m: int, n: int, k: int):
    """The launch bitlinear_forward_lut makes for (M, N, K), or None where it does not apply."""
    out = (ctypes.c_int32 * 6)()
    st = lib().bitlinear_forward_lut_plan(m, n, k, out)
    if st == BL_ERR_UNSUPPORTED:
        return None
    _check("bitlinear_forward_lut_plan", st)
    return _plan_dict(out)


def forward_lut(packed, gamma, xq, absmax, n: int, k: int, y=None, acc=None, want_y: bool = True,
                want_acc: bool = False):
    """bitlinear_forward computed by table lookups (comparison variant, M <= 4)."""
    import torch

    for t, name in ((packed, "packed"), (gamma, "gamma"), (xq, "xq"), (absmax, "absmax")):
        _require_cuda(t, name)
    m = xq.shape[0]
    dev = xq.device
    if want_y and y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    _check("bitlinear_forward_lut", lib().bitlinear_forward_lut(
        packed.data_ptr(), gamma.data_ptr(), xq.data_ptr(), absmax.data_ptr(), m, n, k,
        y.data_ptr() if y is not None else None, acc.data_ptr() if acc is not None else None, _stream(dev)))
    if want_y and want_acc:
        return y, acc
    return y if want_y else acc


def forward_fused(packed, gamma, x, n: int, k: int, y=None, acc=None, xq=None, absmax=None, want_y: bool = True,
                  want_acc: bool = False):
    """Quantise x[M][K] (fp32/bf16) per token and apply the packed weights in one call.

    Returns (y and/or acc, xq, absmax)."""
    import torch

    for t, name in ((packed, "packed"), (gamma, "gamma"), (x, "x")):
        _require_cuda(t, name)
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [tokens, K]")
    if x.dtype == torch.float32:
        dt = BL_F32
    elif x.dtype == torch.bfloat16:
        dt = BL_BF16
    else:
        raise ValueError("x must be float32 or bfloat16")
    m = x.shape[0]
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k_pad(k)), dtype=torch.int8, device=dev)
    if absmax is None:
        absmax = torch.empty(m, dtype=torch.float32, device=dev)
    if want_y and y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    _check("bitlinear_forward_fused", lib().bitlinear_forward_fused(
        packed.data_ptr(), gamma.data_ptr(), x.data_ptr(), dt, m, n, k,
        y.data_ptr() if y is not None else None, acc.data_ptr() if acc is not None else None,
        xq.data_ptr(), absmax.data_ptr(), _stream(dev)))
    out = (y, acc) if (want_y and want_acc) else (y if want_y else acc)
    return out, xq, absmax


def _group_array(mats):
    """Host bl_matrix array for [(packed, gamma, n, y, acc), ...] (y / acc may be None)."""
    if not 1 <= len(mats) <= MAX_GROUP:
        raise ValueError(f"a group holds 1..{MAX_GROUP} matrices")
    arr = (BlMatrix * len(mats))()
    for i, (packed, gamma, n, y, acc) in enumerate(mats):
        for t, name in ((packed, "packed"), (gamma, "gamma")):
            _require_cuda(t, name)
        arr[i] = BlMatrix(packed.data_ptr(), gamma.data_ptr(), n, y.data_ptr() if y is not None else None,
                          acc.data_ptr() if acc is not None else None)
    return arr


def forward_grouped(mats, x, k: int, xq=None, absmax=None, want_y: bool = True, want_acc: bool = False):
    """Several projections of one input x[M][K] (fp32/bf16): ``mats`` is a list of
    (packed, gamma, n).  The activations are quantised once.  Returns (outs, xq, absmax)
    with outs[i] = y_i, acc_i or (y_i, acc_i) as for forward_fused."""
    import torch

    _require_cuda(x, "x")
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [tokens, K]")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    dt = BL_BF16 if x.dtype == torch.bfloat16 else BL_F32
    m = x.shape[0]
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k_pad(k)), dtype=torch.int8, device=dev)
    if absmax is None:
        absmax = torch.empty(m, dtype=torch.float32, device=dev)
    full, outs = [], []
    for packed, gamma, n in mats:
        y = torch.empty((m, n), dtype=torch.float32, device=dev) if want_y else None
        acc = torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None
        full.append((packed, gamma, n, y, acc))
        outs.append((y, acc) if (want_y and want_acc) else (y if want_y else acc))
    arr = _group_array(full)
    _check("bitlinear_forward_grouped", lib().bitlinear_forward_grouped(
        ctypes.addressof(arr), len(full), x.data_ptr(), dt, m, k, xq.data_ptr(), absmax.data_ptr(), _stream(dev)))
    return outs, xq, absmax


def _acts_dtype(x, k=None) -> int:
    import torch

    _require_cuda(x, "x")
    if x.dim() != 2 or (k is not None and x.shape[1] != k):
        raise ValueError("x must be 2-D [tokens, K]")
    if x.dtype == torch.float32:
        return BL_F32
    if x.dtype == torch.bfloat16:
        return BL_BF16
    raise ValueError("x must be float32 or bfloat16")


def _gain_ptr(gain, k: int):
    import torch

    if gain is None:
        return None
    _require_cuda(gain, "gain")
    if gain.dtype != torch.float32 or gain.dim() != 1 or gain.shape[0] != k or not gain.is_contiguous():
        raise ValueError("gain must be a contiguous float32 [K] tensor")
    return gain.data_ptr()


def subln_quantize_acts(x, gain=None, eps: float = 1e-5, xq=None, scale=None):
    """Sub-layer RMS normalisation (per-feature gain, eps) fused with the per-token absmax
    int8 quantiser.  Returns ``(xq int8 [M][K_pad], scale fp32 [M])``; scale is the
    absmax of the normalised row and takes the place of absmax in ``forward``."""
    import torch

    dt = _acts_dtype(x)
    m, k = x.shape
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k_pad(k)), dtype=torch.int8, device=dev)
    if scale is None:
        scale = torch.empty(m, dtype=torch.float32, device=dev)
    _check("bitlinear_subln_quantize_acts", lib().bitlinear_subln_quantize_acts(
        x.data_ptr(), dt, m, k, _gain_ptr(gain, k), eps, xq.data_ptr(), scale.data_ptr(), _stream(dev)))
    return xq, scale


def forward_subln(packed, gamma, x, n: int, k: int, gain=None, eps: float = 1e-5, y=None, acc=None, xq=None,
                  scale=None, want_y: bool = True, want_acc: bool = False):
    """Sub-layer normalisation, quantisation and the packed-weight product in one call.
    Returns (y and/or acc, xq, scale) as forward_fused."""
    import torch

    for t, name in ((packed, "packed"), (gamma, "gamma")):
        _require_cuda(t, name)
    dt = _acts_dtype(x, k)
    m = x.shape[0]
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k_pad(k)), dtype=torch.int8, device=dev)
    if scale is None:
        scale = torch.empty(m, dtype=torch.float32, device=dev)
    if want_y and y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    _check("bitlinear_forward_subln", lib().bitlinear_forward_subln(
        packed.data_ptr(), gamma.data_ptr(), x.data_ptr(), dt, m, n, k, _gain_ptr(gain, k), eps,
        y.data_ptr() if y is not None else None, acc.data_ptr() if acc is not None else None,
        xq.data_ptr(), scale.data_ptr(), _stream(dev)))
    out = (y, acc) if (want_y and want_acc) else (y if want_y else acc)
    return out, xq, scale


def forward_grouped_subln(mats, x, k: int, gain=None, eps: float = 1e-5, xq=None, scale=None,
                          want_y: bool = True, want_acc: bool = False):
    """forward_grouped behind the sub-layer normalisation: one normalising quantisation,
    shared by every matrix.  Returns (outs, xq, scale)."""
    import torch

    dt = _acts_dtype(x, k)
    m = x.shape[0]
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k_pad(k)), dtype=torch.int8, device=dev)
    if scale is None:
        scale = torch.empty(m, dtype=torch.float32, device=dev)
    full, outs = [], []
    for packed, gamma, n in mats:
        y = torch.empty((m, n), dtype=torch.float32, device=dev) if want_y else None
        acc = torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None
        full.append((packed, gamma, n, y, acc))
        outs.append((y, acc) if (want_y and want_acc) else (y if want_y else acc))
    arr = _group_array(full)
    _check("bitlinear_forward_grouped_subln", lib().bitlinear_forward_grouped_subln(
        ctypes.addressof(arr), len(full), x.data_ptr(), dt, m, k, _gain_ptr(gain, k), eps, xq.data_ptr(),
        scale.data_ptr(), _stream(dev)))
    return outs, xq, scale


def forward_gated_relu2(gate, up, x, n: int, k: int, subln: bool = False, gain=None, eps: float = 1e-5, h=None,
                        xq=None, scale=None, workspace=None):
    """Gate / up pair of one input with the squared-ReLU gating: ``gate`` and ``up`` are
    (packed, gamma) of two N x K matrices.  Returns (h fp32 [M][N], xq, scale)."""
    import torch

    for t, name in ((gate[0], "gate packed"), (gate[1], "gate gamma"), (up[0], "up packed"), (up[1], "up gamma")):
        _require_cuda(t, name)
    dt = _acts_dtype(x, k)
    m = x.shape[0]
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k_pad(k)), dtype=torch.int8, device=dev)
    if scale is None:
        scale = torch.empty(m, dtype=torch.float32, device=dev)
    if h is None:
        h = torch.empty((m, n), dtype=torch.float32, device=dev)
    fused = forward_gated_relu2_plan(m, n, k, "bf16" if dt == BL_BF16 else "f32", subln)["kernel"] == "fused"
    fused = fused and x.data_ptr() % 16 == 0 and (not subln or gain is None or gain.data_ptr() % 16 == 0)
    if workspace is None and not fused:
        workspace = torch.empty(int(lib().bitlinear_gated_relu2_workspace_bytes(m, n)), dtype=torch.uint8,
                                device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("bitlinear_forward_gated_relu2", lib().bitlinear_forward_gated_relu2(
        gate[0].data_ptr(), gate[1].data_ptr(), up[0].data_ptr(), up[1].data_ptr(), x.data_ptr(), dt, m, n, k,
        int(subln), _gain_ptr(gain, k) if subln else None, eps, h.data_ptr(), xq.data_ptr(), scale.data_ptr(),
        ws_ptr, ws_len, _stream(dev)))
    return h, xq, scale


def probe_stream(buf, out=None):
    """Read the uint8 device tensor ``buf`` with the decode access pattern (measurement
    probe); returns the per-32-KiB-block XOR checksums (uint32 device tensor)."""
    import torch

    _require_cuda(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    words = int(lib().bitlinear_probe_stream_words(nbytes))
    if words < 0:
        raise ValueError("probe_stream needs a multiple of 1024 bytes")
    if out is None:
        out = torch.empty(words, dtype=torch.int32, device=buf.device)
    _check("bitlinear_probe_stream", lib().bitlinear_probe_stream(buf.data_ptr(), nbytes, out.data_ptr(),
                                                                  out.numel(), _stream(buf.device)))
    return out


def probe_read(buf, workgroups: int, nontemporal: bool = True, out=None):
    """Read the device tensor ``buf`` with a plain grid-stride loop of ``workgroups`` x 256
    lanes (measurement probe); returns the per-workgroup XOR checksums (int32 device tensor)."""
    import torch

    _require_cuda(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(workgroups, dtype=torch.int32, device=buf.device)
    if out.numel() < workgroups:
        raise ValueError("out needs one word per workgroup")
    _check("bitlinear_probe_read", lib().bitlinear_probe_read(buf.data_ptr(), nbytes, workgroups, int(nontemporal),
                                                              out.data_ptr(), _stream(buf.device)))
    return out


def probe_mfma(iters: int, workgroups: int, out):
    """Matrix-core probe: workgroups x 4 waves x 16 independent int8 MFMAs per iteration."""
    _require_cuda(out, "out")
    if out.numel() < workgroups:
        raise ValueError("out needs one word per workgroup")
    _check("bitlinear_probe_mfma", lib().bitlinear_probe_mfma(iters, workgroups, out.data_ptr(), _stream(out.device)))
    return out


def prefill_occupancy() -> dict:
    """Resident workgroups per compute unit of the one-group prefill kernels, from the HIP
    runtime: {"whole": {256: n, 192: n}, "split": {256: n, 192: n}} by tile width."""
    out = (ctypes.c_int32 * 4)()
    _check("bitlinear_probe_prefill_occupancy", lib().bitlinear_probe_prefill_occupancy(out))
    return {"whole": {256: out[0], 192: out[1]}, "split": {256: out[2], 192: out[3]}}


class PreparedCall:
    """One C-ABI call with its arguments marshalled once: raw device pointers, sizes and the
    stream handle, converted to ctypes values up front.  Calling it re-issues the same
    launch for the cost of one foreign call, for launch loops where the per-call Python
    work of the functions above would take longer than the kernel itself.  The caller keeps
    the tensors the pointers came from alive.  The stream is the one current when the call
    was prepared: to record the call into a HIP graph, prepare it inside the capture."""

    def __init__(self, fn: str, *args):
        self._name = fn
        self._fn = getattr(lib(), fn)
        self._args = tuple(t(a) for t, a in zip(self._fn.argtypes, args))
        if len(self._args) != len(self._fn.argtypes):
            raise ValueError(f"{fn} takes {len(self._fn.argtypes)} arguments")

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != BL_OK:
            _check(self._name, st)


def prepare_forward_fused(packed, gamma, x, n: int, k: int, y, xq, absmax) -> PreparedCall:
    """bitlinear_forward_fused on these tensors (y fp32 output), marshalled once."""
    import torch

    for t, name in ((packed, "packed"), (gamma, "gamma"), (x, "x"), (y, "y"), (xq, "xq"), (absmax, "absmax")):
        _require_cuda(t, name)
    dt = BL_BF16 if x.dtype == torch.bfloat16 else BL_F32
    return PreparedCall("bitlinear_forward_fused", packed.data_ptr(), gamma.data_ptr(), x.data_ptr(), dt,
                        x.shape[0], n, k, y.data_ptr(), None, xq.data_ptr(), absmax.data_ptr(), _stream(x.device))


def prepare_forward_grouped(mats, x, k: int, xq, absmax) -> PreparedCall:
    """bitlinear_forward_grouped on these tensors: ``mats`` is a list of
    (packed, gamma, n, y) with fp32 outputs y, marshalled once."""
    import torch

    for t, name in ((x, "x"), (xq, "xq"), (absmax, "absmax")):
        _require_cuda(t, name)
    arr = _group_array([(pk, g, n, y, None) for pk, g, n, y in mats])
    dt = BL_BF16 if x.dtype == torch.bfloat16 else BL_F32
    call = PreparedCall("bitlinear_forward_grouped", ctypes.addressof(arr), len(mats), x.data_ptr(), dt,
                        x.shape[0], k, xq.data_ptr(), absmax.data_ptr(), _stream(x.device))
    call._keep = arr  # the host descriptor array must outlive the call object
    return call


def prepare_forward_subln(packed, gamma, x, n: int, k: int, gain, eps: float, y, xq, scale) -> PreparedCall:
    """bitlinear_forward_subln on these tensors (y fp32 output), marshalled once."""
    for t, name in ((packed, "packed"), (gamma, "gamma"), (y, "y"), (xq, "xq"), (scale, "scale")):
        _require_cuda(t, name)
    dt = _acts_dtype(x, k)
    return PreparedCall("bitlinear_forward_subln", packed.data_ptr(), gamma.data_ptr(), x.data_ptr(), dt,
                        x.shape[0], n, k, _gain_ptr(gain, k), eps, y.data_ptr(), None, xq.data_ptr(),
                        scale.data_ptr(), _stream(x.device))


def prepare_forward_grouped_subln(mats, x, k: int, gain, eps: float, xq, scale) -> PreparedCall:
    """bitlinear_forward_grouped_subln on these tensors: ``mats`` is a list of
    (packed, gamma, n, y) with fp32 outputs y, marshalled once."""
    for t, name in ((xq, "xq"), (scale, "scale")):
        _require_cuda(t, name)
    dt = _acts_dtype(x, k)
    arr = _group_array([(pk, g, n, y, None) for pk, g, n, y in mats])
    call = PreparedCall("bitlinear_forward_grouped_subln", ctypes.addressof(arr), len(mats), x.data_ptr(), dt,
                        x.shape[0], k, _gain_ptr(gain, k), eps, xq.data_ptr(), scale.data_ptr(), _stream(x.device))
    call._keep = arr
    return call


def prepare_subln_quantize_acts(x, gain, eps: float, xq, scale) -> PreparedCall:
    """bitlinear_subln_quantize_acts on these tensors, marshalled once."""
    for t, name in ((xq, "xq"), (scale, "scale")):
        _require_cuda(t, name)
    dt = _acts_dtype(x)
    return PreparedCall("bitlinear_subln_quantize_acts", x.data_ptr(), dt, x.shape[0], x.shape[1],
                        _gain_ptr(gain, x.shape[1]), eps, xq.data_ptr(), scale.data_ptr(), _stream(x.device))


def prepare_forward_gated_relu2(gate, up, x, n: int, k: int, subln: bool, gain, eps: float, h, xq, scale,
                                workspace=None) -> PreparedCall:
    """bitlinear_forward_gated_relu2 on these tensors, marshalled once."""
    for t, name in ((h, "h"), (xq, "xq"), (scale, "scale")):
        _require_cuda(t, name)
    dt = _acts_dtype(x, k)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return PreparedCall("bitlinear_forward_gated_relu2", gate[0].data_ptr(), gate[1].data_ptr(), up[0].data_ptr(),
                        up[1].data_ptr(), x.data_ptr(), dt, x.shape[0], n, k, int(subln),
                        _gain_ptr(gain, k) if subln else None, eps, h.data_ptr(), xq.data_ptr(), scale.data_ptr(),
                        ws_ptr, ws_len, _stream(x.device))


def prepare_forward_lut(packed, gamma, xq, absmax, n: int, k: int, y) -> PreparedCall:
    """bitlinear_forward_lut on these tensors (y fp32 output), marshalled once."""
    for t, name in ((packed, "packed"), (gamma, "gamma"), (xq, "xq"), (absmax, "absmax"), (y, "y")):
        _require_cuda(t, name)
    return PreparedCall("bitlinear_forward_lut", packed.data_ptr(), gamma.data_ptr(), xq.data_ptr(), absmax.data_ptr(),
                        xq.shape[0], n, k, y.data_ptr(), None, _stream(xq.device))


def prepare_forward_binary(packed, beta, xq, absmax, n: int, k: int, y) -> PreparedCall:
    """bitlinear_forward_binary on these tensors (y fp32 output), marshalled once."""
    for t, name in ((packed, "packed"), (beta, "beta"), (xq, "xq"), (absmax, "absmax"), (y, "y")):
        _require_cuda(t, name)
    return PreparedCall("bitlinear_forward_binary", packed.data_ptr(), beta.data_ptr(), xq.data_ptr(),
                        absmax.data_ptr(), xq.shape[0], n, k, y.data_ptr(), None, _stream(xq.device))


def prepare_quantize_acts(x, xq, absmax) -> PreparedCall:
    """bitlinear_quantize_acts on these tensors, marshalled once."""
    import torch

    for t, name in ((x, "x"), (xq, "xq"), (absmax, "absmax")):
        _require_cuda(t, name)
    dt = BL_BF16 if x.dtype == torch.bfloat16 else BL_F32
    return PreparedCall("bitlinear_quantize_acts", x.data_ptr(), dt, x.shape[0], x.shape[1], xq.data_ptr(),
                        absmax.data_ptr(), None, _stream(x.device))


def prepare_forward_ws(packed, gamma, xq, absmax, n: int, k: int, y, workspace) -> PreparedCall:
    """bitlinear_forward_ws on these tensors (y fp32 output), marshalled once."""
    for t, name in ((packed, "packed"), (gamma, "gamma"), (xq, "xq"), (absmax, "absmax"), (y, "y")):
        _require_cuda(t, name)
    return PreparedCall("bitlinear_forward_ws", packed.data_ptr(), gamma.data_ptr(), xq.data_ptr(), absmax.data_ptr(),
                        xq.shape[0], n, k, y.data_ptr(), None,
                        workspace.data_ptr() if workspace is not None else None,
                        workspace.numel() * workspace.element_size() if workspace is not None else 0,
                        _stream(xq.device))


def prepare_forward(packed, gamma, xq, absmax, n: int, k: int, y) -> PreparedCall:
    """bitlinear_forward on these tensors (y fp32 output), marshalled once."""
    for t, name in ((packed, "packed"), (gamma, "gamma"), (xq, "xq"), (absmax, "absmax"), (y, "y")):
        _require_cuda(t, name)
    return PreparedCall("bitlinear_forward", packed.data_ptr(), gamma.data_ptr(), xq.data_ptr(), absmax.data_ptr(),
                        xq.shape[0], n, k, y.data_ptr(), None, _stream(xq.device))


class BitLinear:
    """Inference-time BitLinear: weights quantised once, forward per token batch."""

    def __init__(self, W):
        self.n, self.k = W.shape
        self.packed, self.gamma = quantize_weights(W)

    def __call__(self, x):
        y, _, _ = forward_fused(self.packed, self.gamma, x.contiguous(), self.n, self.k)
        return y
