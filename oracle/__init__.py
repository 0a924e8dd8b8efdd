"""CPU oracle for the BitNet b1.58 BitLinear forward.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path (``bitlinear_fwd_amd``) never imports it,
and the two share no code: the oracle is plain scalar C (``bitlinear_oracle.c``) with a
thin ctypes layer and the exact rational rounding of the mean below, written from the
pages:

* aratech.ae, "BitNet b1.58: Microsoft's 1-bit LLM that runs a 100B model on one CPU",
  section "The solution: BitNet b1.58", sub-sections "Ternary weights {-1, 0, +1}"
  (absmean scale, ``clamp(-1, 1)(round(W * scale_w))``) and "BitLinear: the building
  block" (per-token absmax int8 activations, largest magnitude mapped to 127).
* bhfrc.com news 56965 (BitNet b1.58 on Windows), section 1.1 (ternary x activation is
  add / subtract / nothing) and section 4.1 (2-bit code table 00/01/10/11).

Every function here has a pin in ``tests/test_oracle_pins.py`` (closed forms, brute
force on tiny inputs, invariants, hand-derived golden bytes).  Parity is pinned for
every function except the choices the pages leave open, which are fixed by reading
(round-half-to-even, exact mean, the packed layout, the rescale order); those readings
are listed with the design notes.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# Plain C, no fast-math, no FMA contraction, no target-specific vector code.
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]

_lib = None


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (the checker is built, not used, by build())."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_SRC) > os.path.getmtime(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.orc_n_pad.restype = i64
        lib.orc_n_pad.argtypes = [i64]
        lib.orc_k_pad.restype = i64
        lib.orc_k_pad.argtypes = [i64]
        lib.orc_packed_bytes.restype = i64
        lib.orc_packed_bytes.argtypes = [i64, i64]
        lib.orc_sum_limbs.restype = ctypes.c_int
        lib.orc_sum_limbs.argtypes = []
        lib.orc_abs_sum_fixed.restype = ctypes.c_int
        lib.orc_abs_sum_fixed.argtypes = [p, i64, p]
        lib.orc_ternarise.restype = None
        lib.orc_ternarise.argtypes = [p, i64, ctypes.c_float, p]
        lib.orc_pack.restype = ctypes.c_int
        lib.orc_pack.argtypes = [p, i64, i64, p]
        lib.orc_unpack_codes.restype = None
        lib.orc_unpack_codes.argtypes = [p, i64, i64, p]
        lib.orc_unpack.restype = ctypes.c_int
        lib.orc_unpack.argtypes = [p, i64, i64, p]
        lib.orc_bf16_to_f32.restype = None
        lib.orc_bf16_to_f32.argtypes = [p, i64, p]
        lib.orc_quant_acts.restype = None
        lib.orc_quant_acts.argtypes = [p, i64, i64, p, p]
        lib.orc_subln_quant_acts.restype = None
        lib.orc_subln_quant_acts.argtypes = [p, i64, i64, p, ctypes.c_double, p, p, p]
        lib.orc_gated_relu2.restype = None
        lib.orc_gated_relu2.argtypes = [p, p, i64, p]
        lib.orc_kb_pad.restype = i64
        lib.orc_kb_pad.argtypes = [i64]
        lib.orc_packed_bytes_binary.restype = i64
        lib.orc_packed_bytes_binary.argtypes = [i64, i64]
        lib.orc_binarise.restype = None
        lib.orc_binarise.argtypes = [p, i64, p]
        lib.orc_pack_binary.restype = ctypes.c_int
        lib.orc_pack_binary.argtypes = [p, i64, i64, p]
        lib.orc_unpack_binary.restype = None
        lib.orc_unpack_binary.argtypes = [p, i64, i64, p]
        lib.orc_matmul.restype = ctypes.c_int
        lib.orc_matmul.argtypes = [p, p, i64, i64, i64, i64, p]
        lib.orc_rescale.restype = None
        lib.orc_rescale.argtypes = [p, i64, i64, ctypes.c_float, p, p]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ----------------------------------------------------------------------------- sizes
def n_pad(n: int) -> int:
    return int(_load().orc_n_pad(n))


def k_pad(k: int) -> int:
    return int(_load().orc_k_pad(k))


def packed_bytes(n: int, k: int) -> int:
    return int(_load().orc_packed_bytes(n, k))


# ----------------------------------------------------------------------------- gamma
def round_rational_to_f32(num: int, den: int) -> np.float32:
    """fp32 nearest to the non-negative rational num/den (ties to even mantissa)."""
    if den <= 0 or num < 0:
        raise ValueError("need num >= 0, den > 0")
    if num == 0:
        return np.float32(0.0)
    # Choose e with 2**23 <= num / (den * 2**e) < 2**24: m is then a 24-bit significand.
    e = num.bit_length() - den.bit_length() - 24
    while True:
        n2, d2 = (num, den << e) if e >= 0 else (num << -e, den)
        m, rem = divmod(n2, d2)
        if m >= 1 << 24:
            e += 1
        elif m < 1 << 23:
            e -= 1
        else:
            break
    if e < -149:  # below the normal range: fixed quantum 2**-149
        e = -149
        m, rem = divmod(num << 149, den)
        d2 = den
    twice = 2 * rem
    if twice > d2 or (twice == d2 and (m & 1)):
        m += 1
    return np.float32(float(m) * 2.0 ** e)  # m * 2**e is exactly representable


def exact_abs_sum_scaled(w: np.ndarray) -> int:
    """Sum of |w| over all entries as an exact integer in units of 2**-149.

    Every finite fp32 is an integer multiple of 2**-149, so the sum is an integer in
    those units.  orc_abs_sum_fixed adds each weight, in index order, into a fixed-point
    accumulator wide enough that nothing is ever rounded; its limbs become one Python
    integer here."""
    a = np.ascontiguousarray(w, dtype=np.float32).ravel()
    lib = _load()
    limbs = np.zeros(int(lib.orc_sum_limbs()), dtype=np.uint32)
    if lib.orc_abs_sum_fixed(_ptr(a), a.size, _ptr(limbs)) != 0:
        raise ValueError("non-finite weight, or more than 2**40 weights")
    return sum(int(v) << (32 * i) for i, v in enumerate(limbs))


def gamma_absmean(w: np.ndarray) -> np.float32:
    """gamma = mean |W| over the whole tensor, the exact mean rounded to fp32.

    aratech.ae article, "Ternary weights {-1, 0, +1}": the weight scale is the
    reciprocal of the mean absolute value taken over the entire weight tensor."""
    count = int(np.asarray(w).size)
    if count == 0:
        raise ValueError("empty weight tensor")
    return round_rational_to_f32(exact_abs_sum_scaled(w), count << 149)


def gamma_bruteforce(w: np.ndarray) -> np.float32:
    """Slow Fraction-based gamma for tiny tensors (used only by the pins)."""
    vals = np.asarray(w, dtype=np.float32).ravel()
    s = sum((Fraction(abs(float(v))) for v in vals), Fraction(0))
    mean = s / len(vals)
    return round_rational_to_f32(mean.numerator, mean.denominator)


# ----------------------------------------------------------------------------- steps
def ternarise(w: np.ndarray, gamma) -> np.ndarray:
    """Codes q = clamp(rint(fl32(W * fl32(1/gamma))), -1, 1) as int8, same shape as W."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    q = np.empty(w.shape, dtype=np.int8)
    _load().orc_ternarise(_ptr(w), w.size, float(np.float32(gamma)), _ptr(q))
    return q


def pack(q: np.ndarray) -> np.ndarray:
    """Pack ternary q[N][K] into the tiled 2-bit layout (uint8, N_pad*K_pad/4 bytes)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    n, k = q.shape
    out = np.zeros(packed_bytes(n, k), dtype=np.uint8)
    rc = _load().orc_pack(_ptr(q), n, k, _ptr(out))
    if rc != 0:
        raise ValueError("value outside {-1, 0, 1}")
    return out


def unpack_codes(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size == packed_bytes(n, k)
    out = np.empty((n_pad(n), k_pad(k)), dtype=np.uint8)
    _load().orc_unpack_codes(_ptr(packed), n, k, _ptr(out))
    return out


def unpack(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size == packed_bytes(n, k)
    out = np.empty((n, k), dtype=np.int8)
    if _load().orc_unpack(_ptr(packed), n, k, _ptr(out)) != 0:
        raise ValueError("padding code inside the matrix")
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    _load().orc_bf16_to_f32(_ptr(bits), bits.size, _ptr(out))
    return out


def quant_acts(x: np.ndarray):
    """Per-token absmax int8: returns (xq [M][K_pad] int8, absmax [M] fp32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    m, k = x.shape
    xq = np.empty((m, k_pad(k)), dtype=np.int8)
    a = np.empty(m, dtype=np.float32)
    _load().orc_quant_acts(_ptr(x), m, k, _ptr(xq), _ptr(a))
    return xq, a


def subln_quant_acts(x: np.ndarray, gain=None, eps: float = 1e-5):
    """Sub-layer RMS normalisation, then per-token absmax int8 (orc_subln_quant_acts).

    Returns (xq [M][K_pad] int8, scale [M] fp32, scale64 [M] fp64, h_absmax [M] fp32):
    the codes, the dequantisation scale max|n| rounded to fp32 and in fp64, and the
    absmax of h = fl32(x * gain) on which the codes were decided.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    m, k = x.shape
    xq = np.empty((m, k_pad(k)), dtype=np.int8)
    ha = np.empty(m, dtype=np.float32)
    sc = np.empty(m, dtype=np.float64)
    g = None
    if gain is not None:
        g = np.ascontiguousarray(gain, dtype=np.float32)
        assert g.shape == (k,)
    if not (eps >= 0.0 and math.isfinite(eps)):
        raise ValueError("eps must be finite and >= 0")
    _load().orc_subln_quant_acts(_ptr(x), m, k, None if g is None else _ptr(g), float(np.float32(eps)),
                                 _ptr(xq), _ptr(ha), _ptr(sc))
    return xq, sc.astype(np.float32), sc, ha


def matmul(q: np.ndarray, xq: np.ndarray, k: int) -> np.ndarray:
    """acc[m][n] = sum_{k' < k} xq[m][k'] * q[n][k'] in exact integers (int32 result)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    n = q.shape[0]
    m = xq.shape[0]
    assert q.shape[1] == k and xq.shape[1] >= k
    acc = np.empty((m, n), dtype=np.int32)
    if _load().orc_matmul(_ptr(q), _ptr(xq), m, n, k, xq.shape[1], _ptr(acc)) != 0:
        raise OverflowError("accumulator exceeds int32")
    return acc


def rescale(acc: np.ndarray, gamma, absmax: np.ndarray) -> np.ndarray:
    """y = acc * gamma * absmax[m] / 127 in fp64."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    absmax = np.ascontiguousarray(absmax, dtype=np.float32)
    m, n = acc.shape
    y = np.empty((m, n), dtype=np.float64)
    _load().orc_rescale(_ptr(acc), m, n, float(np.float32(gamma)), _ptr(absmax), _ptr(y))
    return y


# ----------------------------------------------------------------------------- whole path
def quantize_weights(w: np.ndarray):
    """(gamma, q [N][K] int8, packed uint8) for latent weights W[N][K] (out x in)."""
    g = gamma_absmean(w)
    q = ternarise(w, g)
    return g, q, pack(q)


def forward(q: np.ndarray, gamma, xq: np.ndarray, absmax: np.ndarray, k: int):
    """(acc int32 [M][N], y float64 [M][N]) from ternary codes and quantised activations."""
    acc = matmul(q, xq, k)
    return acc, rescale(acc, gamma, absmax)


def gated_relu2(y_gate: np.ndarray, y_up: np.ndarray) -> np.ndarray:
    """Squared-ReLU gating of a gate / up pair: relu(y_gate)^2 * y_up in fp64."""
    g = np.ascontiguousarray(y_gate, dtype=np.float64)
    u = np.ascontiguousarray(y_up, dtype=np.float64)
    assert g.shape == u.shape
    h = np.empty(g.shape, dtype=np.float64)
    _load().orc_gated_relu2(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def ffn_gate_up(q_gate: np.ndarray, gamma_gate, q_up: np.ndarray, gamma_up, xq: np.ndarray, absmax: np.ndarray,
                k: int) -> np.ndarray:
    """h [M][N] fp64 of the gate / up pair on quantised activations: two forwards, then gating."""
    _, y_g = forward(q_gate, gamma_gate, xq, absmax, k)
    _, y_u = forward(q_up, gamma_up, xq, absmax, k)
    return gated_relu2(y_g, y_u)


# ----------------------------------------------------------------------------- binary variant
def kb_pad(k: int) -> int:
    return int(_load().orc_kb_pad(k))


def packed_bytes_binary(n: int, k: int) -> int:
    return int(_load().orc_packed_bytes_binary(n, k))


def binarise(w: np.ndarray) -> np.ndarray:
    """sign(W) in {-1, +1} with +1 for W >= 0 (lpnh.cn section 2.1)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    q = np.empty(w.shape, dtype=np.int8)
    _load().orc_binarise(_ptr(w), w.size, _ptr(q))
    return q


def pack_binary(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    n, k = q.shape
    out = np.empty(packed_bytes_binary(n, k), dtype=np.uint8)
    if _load().orc_pack_binary(_ptr(q), n, k, _ptr(out)) != 0:
        raise ValueError("binary codes must be -1 or +1")
    return out


def unpack_binary(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size == packed_bytes_binary(n, k)
    out = np.empty((n, k), dtype=np.int8)
    _load().orc_unpack_binary(_ptr(packed), n, k, _ptr(out))
    return out


def quantize_weights_binary(w: np.ndarray):
    """(beta, q [N][K] in {-1, +1}, packed) for latent weights W[N][K]; beta = mean |W|."""
    beta = gamma_absmean(w)
    q = binarise(w)
    return beta, q, pack_binary(q)
