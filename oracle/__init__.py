"""CPU oracle for quantized-KV decode attention (numpy front end to kvq_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does, and
this package never imports the product.  See kvq_oracle.c for what each
function computes and which page passage defines it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkvq_oracle.so")

INT8, INT4, FP8 = 1, 2, 3
BF16 = 4  # unquantized cache: the codes are the bf16 values, no scales
PER_ROW, PER_TENSOR, PER_CHANNEL = 1, 2, 3
QMAX = {INT8: 127.0, INT4: 7.0, FP8: 448.0}


def build(force: bool = True) -> str:
    """Compile kvq_oracle.c with gcc (IEEE arithmetic: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        P, I, F, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
        L.kvo_bf16_to_float.argtypes = [ctypes.c_uint16]
        L.kvo_bf16_to_float.restype = F
        L.kvo_fp8_decode.argtypes = [ctypes.c_uint8]
        L.kvo_fp8_decode.restype = D
        L.kvo_fp8_encode.argtypes = [F]
        L.kvo_fp8_encode.restype = ctypes.c_uint8
        L.kvo_row_bytes.argtypes = [I, I]
        L.kvo_row_bytes.restype = I
        L.kvo_quantize_row.argtypes = [P, I, I, I, P, P, P]
        L.kvo_quantize_row.restype = None
        L.kvo_dequantize_row.argtypes = [P, I, I, I, F, P, P]
        L.kvo_dequantize_row.restype = None
        L.kvo_append.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, I, I, P, P, I]
        L.kvo_append.restype = None
        L.kvo_dequantize.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, I, P, P, I, I, P, P]
        L.kvo_dequantize.restype = None
        L.kvo_attend.argtypes = [P, P, P, I, I, I, I, I, I, P, F, P, P, P]
        L.kvo_attend.restype = None
        L.kvo_attend_ex.argtypes = [P, P, P, I, I, I, I, I, I, P, F, P, F, I, P, P]
        L.kvo_attend_ex.restype = None
        L.kvo_attend_ex2.argtypes = [P, P, P, I, I, I, I, I, I, P, F, P, F, I, P, P, P]
        L.kvo_attend_ex2.restype = None
        L.kvo_cache_bytes_per_token.argtypes = [I, I, I, I, I]
        L.kvo_cache_bytes_per_token.restype = D
        L.kvo_num_threads.argtypes = []
        L.kvo_num_threads.restype = I
        L.kvo_set_num_threads.argtypes = [I]
        L.kvo_set_num_threads.restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def row_bytes(dtype: int, D: int) -> int:
    return D // 2 if dtype == INT4 else 2 * D if dtype == BF16 else D


# ------------------------------------------------------------------ codecs

def fp8_decode(codes: np.ndarray) -> np.ndarray:
    f = lib().kvo_fp8_decode
    return np.array([f(int(c)) for c in np.asarray(codes, np.uint8).ravel()],
                    np.float64).reshape(np.shape(codes))


def fp8_encode(y: np.ndarray) -> np.ndarray:
    f = lib().kvo_fp8_encode
    y = np.asarray(y, np.float32)
    return np.array([f(float(v)) for v in y.ravel()], np.uint8).reshape(y.shape)


def quantize_rows(x_bits: np.ndarray, dtype: int, mode: int, static_scale=None):
    """Quantize rows of bf16 bit patterns ``[N, D]`` (uint16).

    Returns (codes [N, row_bytes] uint8, scales [N] fp32; zeros for static modes).
    ``static_scale`` is fp32 [1] (per-tensor) or [D] (per-channel, this head).
    """
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    N, D = x_bits.shape
    codes = np.zeros((N, row_bytes(dtype, D)), np.uint8)
    scales = np.zeros(N, np.float32)
    ss = _c(static_scale, np.float32)
    L = lib()
    for i in range(N):
        L.kvo_quantize_row(_p(x_bits[i]), D, dtype, mode, _p(ss), _p(codes[i]),
                           ctypes.c_void_p(scales.ctypes.data + 4 * i))
    return codes, scales


def dequantize_rows(codes: np.ndarray, D: int, dtype: int, mode: int, scales=None,
                    static_scale=None) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    N = codes.shape[0]
    out = np.zeros((N, D), np.float32)
    ss = _c(static_scale, np.float32)
    L = lib()
    for i in range(N):
        s = float(scales[i]) if scales is not None else 0.0
        L.kvo_dequantize_row(_p(codes[i]), D, dtype, mode, s, _p(ss), _p(out[i]))
    return out


# ------------------------------------------------------------------ cache

class Cache:
    """Host-side quantized cache: codes [num_blocks, Hkv, bs, row_bytes] uint8 and,
    for per-row scales, scales [num_blocks, Hkv, bs] fp32."""

    def __init__(self, dtype, mode, Hkv, D, block_size, num_blocks, k_static=None,
                 v_static=None, v_mode=None):
        """mode: the K scale mode; v_mode: the V scale mode (default: the same).
        A bf16 cache has no scales (both modes are 0)."""
        if dtype == BF16:
            mode, v_mode = 0, 0
        self.dtype, self.mode, self.Hkv, self.D = dtype, mode, Hkv, D
        self.v_mode = mode if not v_mode else v_mode
        self.block_size, self.num_blocks = block_size, num_blocks
        rb = row_bytes(dtype, D)
        self.k_codes = np.zeros((num_blocks, Hkv, block_size, rb), np.uint8)
        self.v_codes = np.zeros_like(self.k_codes)
        self.k_scales = np.zeros((num_blocks, Hkv, block_size), np.float32)
        self.v_scales = np.zeros_like(self.k_scales)
        self.k_static = _c(k_static, np.float32)
        self.v_static = _c(v_static, np.float32)

    def append(self, k_bits: np.ndarray, v_bits: np.ndarray, positions, block_table=None):
        """k_bits, v_bits: bf16 bit patterns [B, Tn, Hkv, D]."""
        k_bits = np.ascontiguousarray(k_bits, np.uint16)
        v_bits = np.ascontiguousarray(v_bits, np.uint16)
        B, Tn = k_bits.shape[:2]
        pos = np.ascontiguousarray(positions, np.int32)
        bt = _c(block_table, np.int32)
        mb = 0 if bt is None else bt.shape[1]
        lib().kvo_append(self.dtype, self.mode, self.v_mode, self.Hkv, self.D, self.block_size,
                         _p(self.k_codes), _p(self.v_codes), _p(self.k_scales),
                         _p(self.v_scales), _p(self.k_static), _p(self.v_static),
                         _p(k_bits), _p(v_bits), B, Tn, _p(pos), _p(bt), mb)

    def dequantize(self, lens, block_table=None, lmax: Optional[int] = None):
        """Dense fp32 K-hat, V-hat [B, Hkv, Lmax, D] of every sequence."""
        lens = np.ascontiguousarray(lens, np.int32)
        B = lens.shape[0]
        lmax = int(lens.max()) if lmax is None else lmax
        lmax = max(lmax, 1)
        bt = _c(block_table, np.int32)
        mb = 0 if bt is None else bt.shape[1]
        K = np.empty((B, self.Hkv, lmax, self.D), np.float32)
        V = np.empty_like(K)
        lib().kvo_dequantize(self.dtype, self.mode, self.v_mode, self.Hkv, self.D, self.block_size,
                             _p(self.k_codes), _p(self.v_codes), _p(self.k_scales),
                             _p(self.v_scales), _p(self.k_static), _p(self.v_static), B,
                             _p(lens), _p(bt), mb, lmax, _p(K), _p(V))
        return K, V


def attend(q_bits: np.ndarray, K: np.ndarray, V: np.ndarray, lens, scale: float,
           sink: Optional[np.ndarray] = None, Hkv: Optional[int] = None, softcap: float = 0.0,
           window: int = 0, return_max: bool = False):
    """fp64 softmax attention.  q_bits bf16 bits [B, Tq, Hq, D]; K, V fp32
    [B, Hkv, Lmax, D].  softcap > 0 caps every scaled logit as c tanh(z / c);
    window > 0 lets a query at position p see tokens p - window + 1 .. p only.
    Returns (out fp64 [B, Tq, Hq, D], lse fp64 [B, Tq, Hq]), and with
    return_max also the largest logit of each row, fp64 [B, Tq, Hq]."""
    q_bits = np.ascontiguousarray(q_bits, np.uint16)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    B, Tq, Hq, D = q_bits.shape
    hkv = K.shape[1] if Hkv is None else Hkv
    lens = np.ascontiguousarray(lens, np.int32)
    out = np.empty((B, Tq, Hq, D), np.float64)
    lse = np.empty((B, Tq, Hq), np.float64)
    sk = _c(sink, np.float32)
    m = np.empty((B, Tq, Hq), np.float64)
    lib().kvo_attend_ex2(_p(q_bits), _p(K), _p(V), B, Tq, Hq, hkv, D, K.shape[2], _p(lens),
                         float(scale), _p(sk), float(softcap), int(window), _p(out), _p(lse), _p(m))
    return (out, lse, m) if return_max else (out, lse)


def num_threads() -> int:
    return lib().kvo_num_threads()


def set_num_threads(n: int) -> None:
    lib().kvo_set_num_threads(int(n))


def cache_bytes_per_token(bits: int, per_row_scales: bool, layers: int, Hkv: int, D: int) -> float:
    return lib().kvo_cache_bytes_per_token(bits, int(per_row_scales), layers, Hkv, D)


def build_cache(w, lens=None):
    """Quantize every cached row of a workload (see kvq_inputs.Workload) into a
    fresh oracle cache by one bulk append per sequence."""
    import torch  # only for the bf16 bit view of the workload tensors

    c = Cache(w.dtype, w.mode, w.Hkv, w.D, w.block_size, w.num_blocks, w.k_static, w.v_static,
              v_mode=w.v_mode)
    lens = w.lens if lens is None else lens
    kb = w.k.contiguous().view(torch.int16).numpy().view(np.uint16)
    vb = w.v.contiguous().view(torch.int16).numpy().view(np.uint16)
    for b in range(w.B):
        L = int(lens[b])
        if L == 0:
            continue
        # one sequence at a time; a contiguous cache is a table whose only
        # entry for sequence b is block b
        bt = np.array([[b]], np.int32) if w.block_table is None else w.block_table[b:b + 1]
        c.append(kb[b:b + 1, :L], vb[b:b + 1, :L], np.zeros(1, np.int32), bt)
    return c


def reference(w, cache: Optional[Cache] = None):
    """Oracle output of one decode step of workload ``w``: dequantize the cache to
    fp32, then fp64 attention.  Returns (out fp64 [B,Tq,Hq,D], lse, cache)."""
    import torch

    if cache is None:
        cache = build_cache(w)
    K, V = cache.dequantize(w.lens, w.block_table)
    qb = w.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    out, lse = attend(qb, K, V, w.lens, w.sm_scale, w.sink, w.Hkv, w.softcap, w.window)
    return out, lse, cache
