"""Seeded synthetic inputs for the quantized-KV decode workloads.

This module is the only code shared by the CPU oracle's tests and the HIP
path's tests and benchmark.  It draws tensors and metadata; it does not
quantize, dequantize or attend.  The one piece of arithmetic it holds is the
*calibration* of static scales (per-tensor ``amax/448`` for fp8 and
per-channel ``amax/7`` for int4), which is how the caller prepares the scale
inputs that the pages describe as coming from an offline calibration
("[CUDA] PagedAttention: quantized KV cache ...", Summary of Changes, the
k_scale / v_scale inputs; "[CUDA] Add INT4 paged KV cache with per-channel
scales", description of static PER_TENSOR / PER_CHANNEL scales).  The library
under test receives those scales as plain inputs.

Seeding: every tensor of workload ``cfg`` comes from its own CPU
``torch.Generator`` seeded with ``100*cfg + k``, where k = 0 q, 1 K, 2 V,
3 lengths, 4 block permutation, 5 sinks, 6 calibration batch, 7 outlier
channels.  Draws are fp32 ``randn`` cast to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

INT8, INT4, FP8, BF16 = 1, 2, 3, 4
PER_ROW, PER_TENSOR, PER_CHANNEL = 1, 2, 3
DTYPE_NAMES = {"int8": INT8, "int4": INT4, "fp8": FP8, "bf16": BF16}
MODE_NAMES = {"per_row": PER_ROW, "per_tensor": PER_TENSOR, "per_channel": PER_CHANNEL}

SWEEP_CTX = (1024, 4096, 16384, 65536, 262144)


@dataclass
class Workload:
    """One decode step's inputs, all on the CPU.

    k, v hold every row that is appended to build the cache, token-major
    ``[B, Lmax, Hkv, D]`` bf16 (rows past ``lens[b]`` are never appended).
    q is ``[B, Tq, Hq, D]`` bf16.  ``lens[b]`` counts cached tokens including
    the Tq query tokens.  Paged workloads carry ``block_table`` ``[B, max_blocks]``
    int32 into a pool of ``num_blocks`` blocks of ``block_size`` tokens;
    contiguous ones have ``block_table = None``, ``num_blocks = B`` and
    ``block_size = capacity``.
    """

    name: str
    cfg: int
    B: int
    Hq: int
    Hkv: int
    D: int
    Tq: int
    dtype: int
    mode: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    lens: np.ndarray
    block_size: int
    num_blocks: int
    block_table: Optional[np.ndarray]
    k_static: Optional[np.ndarray] = None  # fp32 [1] or [Hkv, D]
    v_static: Optional[np.ndarray] = None
    sink: Optional[np.ndarray] = None  # fp32 [Hq]
    v_mode: int = 0       # the V scale mode when it differs from the K one (0: same)
    softcap: float = 0.0  # > 0: logits capped as softcap * tanh(z / softcap)
    window: int = 0       # > 0: a query at position p sees tokens p - window + 1 .. p
    sm_scale: float = 0.0
    meta: dict = field(default_factory=dict)

    @property
    def lmax(self) -> int:
        return int(self.lens.max()) if self.lens.size else 0

    @property
    def max_blocks(self) -> int:
        return 0 if self.block_table is None else int(self.block_table.shape[1])

    @property
    def row_bytes(self) -> int:
        return self.D // 2 if self.dtype == INT4 else 2 * self.D if self.dtype == BF16 else self.D


def gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def randn_bf16(shape, seed: int) -> torch.Tensor:
    return torch.randn(*shape, generator=gen(seed), dtype=torch.float32).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 numpy array of its bit patterns (no copy of values)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _outlier_scale(shape_hd, n_pairs: int, seed: int) -> torch.Tensor:
    """x8 multiplier on ``n_pairs`` seeded (head, channel) pairs, 1 elsewhere."""
    H, D = shape_hd
    perm = torch.randperm(H * D, generator=gen(seed))[:n_pairs]
    m = torch.ones(H * D, dtype=torch.float32)
    m[perm] = 8.0
    return m.view(H, D)


def _static_per_tensor(x: torch.Tensor, qmax: float) -> np.ndarray:
    amax = np.float32(x.float().abs().max().item())
    return np.array([amax / np.float32(qmax)], dtype=np.float32)


def _static_per_channel(calib: torch.Tensor, qmax: float) -> np.ndarray:
    # calib [Tc, Hkv, D] -> [Hkv, D]
    amax = calib.float().abs().amax(dim=0).numpy().astype(np.float32)
    return (amax / np.float32(qmax)).astype(np.float32)


def _paged_table(B: int, max_blocks: int, seed: int) -> np.ndarray:
    perm = torch.randperm(B * max_blocks, generator=gen(seed)).to(torch.int32)
    return perm.view(B, max_blocks).numpy().copy()


def make_workload(cfg: int, ctx: Optional[int] = None, dtype: Optional[str] = None,
                  B: Optional[int] = None, max_len: Optional[int] = None,
                  Tq: Optional[int] = None, G: Optional[int] = None,
                  Hkv: Optional[int] = None, D: Optional[int] = None) -> Workload:
    """Build the seeded inputs of workload ``cfg`` (1..5).

    cfg 1  tiny decode: B1 Hq4 Hkv1 D64, 256 cached tokens, int8 per-row.
    cfg 2  B1 Hq24 Hkv4 D256, 4096 tokens, 1 % of (head, channel) pairs x8, int8 per-row.
    cfg 3  same geometry, ``ctx`` in SWEEP_CTX, ``dtype`` int8 or int4, per-row.
    (``dtype="bf16"`` gives any of them as an unquantized cache, without scales.)
    cfg 4  paged fp8 per-tensor: B4 Hq32 Hkv8 D128, lengths ~ U[1, 32768], block 16,
           random block table over a shared pool, a head-sink logit per query head.
    cfg 5  paged int4 per-channel speculative decode: B4 Hq24 Hkv4 D256, 32768 prompt
           tokens + 8 query tokens, block 16, per-channel scales from a calibration batch.

    The keyword overrides shrink a workload for tests (``ctx``/``max_len`` bound
    the lengths, ``B``/``Tq``/``G``/``Hkv``/``D`` change the geometry) while
    keeping its value distributions and structure.
    """
    s0 = 100 * cfg
    paged = cfg in (4, 5)
    if cfg == 1:
        b, hkv, g, d, tq = 1, 1, 4, 64, 1
        lens = np.full(1, 256 if ctx is None else ctx, np.int32)
        dt, md = INT8, PER_ROW
    elif cfg in (2, 3):
        b, hkv, g, d, tq = 1, 4, 6, 256, 1
        c = (4096 if cfg == 2 else 65536) if ctx is None else ctx
        lens = np.full(1, c, np.int32)
        dt = DTYPE_NAMES[dtype or "int8"]
        md = PER_ROW
    elif cfg == 4:
        b, hkv, g, d, tq = 4, 8, 4, 128, 1
        dt, md = FP8, PER_TENSOR
    elif cfg == 5:
        b, hkv, g, d, tq = 4, 4, 6, 256, 8
        dt, md = INT4, PER_CHANNEL
    else:
        raise ValueError(f"unknown workload {cfg}")
    if dtype is not None:
        dt = DTYPE_NAMES[dtype]
    if dt == BF16:  # the same workload through an unquantized cache: no scales
        md = 0
    b = B if B is not None else b
    hkv = Hkv if Hkv is not None else hkv
    g = G if G is not None else g
    d = D if D is not None else d
    tq = Tq if Tq is not None else tq
    hq = g * hkv

    if cfg == 4:
        hi = 32768 if max_len is None else max_len
        lens = torch.randint(1, hi + 1, (b,), generator=gen(s0 + 3), dtype=torch.int64)
        lens = lens.numpy().astype(np.int32)
        lens = np.maximum(lens, tq).astype(np.int32)
    elif cfg == 5:
        prompt = 32768 if ctx is None else ctx
        lens = np.full(b, prompt + tq, np.int32)
    elif cfg in (1, 2, 3):
        lens = np.full(b, int(lens[0]), np.int32)

    lmax = int(lens.max())
    q = randn_bf16((b, tq, hq, d), s0 + 0)
    kf = torch.randn(b, lmax, hkv, d, generator=gen(s0 + 1), dtype=torch.float32)
    vf = torch.randn(b, lmax, hkv, d, generator=gen(s0 + 2), dtype=torch.float32)
    meta = {}
    if cfg == 2:
        n_pairs = int(round(0.01 * hkv * d))
        kf = kf * _outlier_scale((hkv, d), n_pairs, s0 + 7)
        vf = vf * _outlier_scale((hkv, d), n_pairs, s0 + 17)
        qm = _outlier_scale((hq, d), int(round(0.01 * hq * d)), s0 + 27)
        q = (q.float() * qm).to(torch.bfloat16)
        meta["outlier_pairs"] = n_pairs
    k = kf.to(torch.bfloat16)
    v = vf.to(torch.bfloat16)
    del kf, vf

    if paged:
        block_size = 16
        max_blocks = (lmax + block_size - 1) // block_size
        if cfg == 4 and max_len is None:
            max_blocks = 32768 // block_size
        table = _paged_table(b, max_blocks, s0 + 4)
        num_blocks = b * max_blocks
    else:
        block_size = max(16, (lmax + 15) // 16 * 16)  # contiguous capacity
        table = None
        num_blocks = b

    k_static = v_static = None
    if md == PER_TENSOR:
        qmax = {INT8: 127.0, INT4: 7.0, FP8: 448.0}[dt]
        # amax over the rows that are actually cached
        kk = torch.cat([k[i, : lens[i]] for i in range(b)])
        vv = torch.cat([v[i, : lens[i]] for i in range(b)])
        k_static = _static_per_tensor(kk, qmax)
        v_static = _static_per_tensor(vv, qmax)
    elif md == PER_CHANNEL:
        qmax = {INT8: 127.0, INT4: 7.0, FP8: 448.0}[dt]
        calib_k = randn_bf16((2048, hkv, d), s0 + 6)
        calib_v = randn_bf16((2048, hkv, d), s0 + 16)
        k_static = _static_per_channel(calib_k, qmax)
        v_static = _static_per_channel(calib_v, qmax)

    sink = None
    if cfg == 4:
        sink = torch.randn(hq, generator=gen(s0 + 5), dtype=torch.float32).numpy()

    sm = np.float32(1.0) / np.float32(math.sqrt(d))
    name = {1: "tiny", 2: "27b-4k-outliers", 3: "27b-sweep", 4: "paged-fp8-sink",
            5: "paged-int4-spec"}[cfg]
    return Workload(name=name, cfg=cfg, B=b, Hq=hq, Hkv=hkv, D=d, Tq=tq, dtype=dt, mode=md,
                    q=q, k=k, v=v, lens=lens, block_size=block_size, num_blocks=num_blocks,
                    block_table=table, k_static=k_static, v_static=v_static, sink=sink,
                    sm_scale=float(sm), meta=meta)


def random_workload(seed: int, B: int, Hkv: int, G: int, D: int, Tq: int, lens,
                    dtype: int, mode: int, block_size: Optional[int] = None,
                    sink: bool = False, softcap: float = 0.0, window: int = 0,
                    v_mode: Optional[int] = None) -> Workload:
    """Small seeded workload of any geometry for property tests."""
    lens = np.asarray(lens, np.int32)
    lmax = int(lens.max()) if lens.size else 0
    hq = G * Hkv
    q = randn_bf16((B, Tq, hq, D), seed + 0)
    k = randn_bf16((B, max(lmax, 1), Hkv, D), seed + 1)
    v = randn_bf16((B, max(lmax, 1), Hkv, D), seed + 2)
    if block_size is None:
        table = None
        bs = max(16, (lmax + 15) // 16 * 16)  # contiguous capacity, a multiple of 16
        nb = B
    else:
        bs = block_size
        mb = max(1, (lmax + bs - 1) // bs)
        table = _paged_table(B, mb, seed + 4)
        nb = B * mb
    if dtype == BF16:  # unquantized: no scales of either side
        mode, v_mode = 0, 0
    qmax = {INT8: 127.0, INT4: 7.0, FP8: 448.0, BF16: 0.0}[dtype]
    vm = mode if v_mode is None else v_mode
    k_static = v_static = None
    if mode == PER_TENSOR:
        k_static = _static_per_tensor(k, qmax)
    elif mode == PER_CHANNEL:
        k_static = _static_per_channel(randn_bf16((256, Hkv, D), seed + 6), qmax)
    if vm == PER_TENSOR:
        v_static = _static_per_tensor(v, qmax)
    elif vm == PER_CHANNEL:
        v_static = _static_per_channel(randn_bf16((256, Hkv, D), seed + 16), qmax)
    sk = torch.randn(hq, generator=gen(seed + 5)).numpy().astype(np.float32) if sink else None
    sm = float(np.float32(1.0) / np.float32(math.sqrt(D)))
    return Workload(name=f"random-{seed}", cfg=0, B=B, Hq=hq, Hkv=Hkv, D=D, Tq=Tq, dtype=dtype,
                    mode=mode, q=q, k=k, v=v, lens=lens, block_size=bs, num_blocks=nb,
                    block_table=table, k_static=k_static, v_static=v_static, sink=sk,
                    sm_scale=sm, softcap=float(np.float32(softcap)), window=int(window),
                    v_mode=0 if vm == mode else vm)
