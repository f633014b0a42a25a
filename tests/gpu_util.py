"""Helpers for the GPU parity tests: run the HIP path through the C ABI on a
seeded workload and compare with the CPU oracle.

Tolerances (kv-quant-attn page, "Correctness": the kernel's residual against
fp32 attention on the dequantized cache is the bf16 output rounding floor):
  codes and per-row scales   bit-exact
  attention output           relative L2 over the whole output <= 2e-3
                             (bf16 rounding of the output alone is ~1.66e-3)
  any single (b, j, h) row   relative L2 <= 4e-3 (a D-element sample of the
                             same rounding floor fluctuates more)
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import kvq_inputs as ki
import oracle
import quantized_kv_cache_02_amd as kvq

REL_TOL = 2e-3
ROW_TOL = 4e-3


def log(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def gpu_cache(w: ki.Workload, device="cuda") -> kvq.KVCache:
    return kvq.KVCache(w.dtype, w.mode, w.Hkv, w.D, w.block_size, w.num_blocks, w.k_static,
                       w.v_static, device=device, v_scale_mode=w.v_mode)


def gpu_build(w: ki.Workload, cache: kvq.KVCache, device="cuda"):
    """Quantize every cached row with kvq_append (one bulk call per sequence)."""
    table = None if w.block_table is None else torch.from_numpy(w.block_table).to(device)
    if table is None:
        # contiguous: one call for all sequences, Lmax rows each (rows past a
        # sequence's length are never read)
        k = w.k.to(device)
        v = w.v.to(device)
        kvq.append(cache, k, v, torch.zeros(w.B, dtype=torch.int32, device=device))
    else:
        for b in range(w.B):
            L = int(w.lens[b])
            if L == 0:
                continue
            k = w.k[b:b + 1, :L].contiguous().to(device)
            v = w.v[b:b + 1, :L].contiguous().to(device)
            kvq.append(cache, k, v, torch.zeros(1, dtype=torch.int32, device=device),
                       table[b:b + 1].contiguous())
    return table


def gpu_decode(w: ki.Workload, cache: kvq.KVCache, table, max_seq_len=None, device="cuda"):
    q = w.q.to(device)
    lens = torch.from_numpy(w.lens).to(device)
    sink = None if w.sink is None else torch.from_numpy(w.sink).to(device)
    msl = max(int(w.lens.max()), 1) if max_seq_len is None else max_seq_len
    if table is None:
        out = kvq.decode_attend(cache, q, lens, msl, w.sm_scale, head_sink=sink)
    else:
        out = kvq.paged_decode_attend(cache, q, lens, msl, w.sm_scale, table, head_sink=sink)
    torch.cuda.synchronize()
    return out


def compare_codes(w: ki.Workload, cache: kvq.KVCache, ocache: oracle.Cache):
    """Bit-exact codes and per-row scales on every row the workload wrote."""
    kc = cache.k_codes.cpu().numpy()
    vc = cache.v_codes.cpu().numpy()
    ks = cache.k_scales.cpu().numpy() if w.mode == ki.PER_ROW else None
    vs = cache.v_scales.cpu().numpy() if (w.v_mode or w.mode) == ki.PER_ROW else None
    for b in range(w.B):
        L = int(w.lens[b])
        if L == 0:
            continue
        if w.block_table is None:
            sel = (b, slice(None), slice(0, L))
            pairs = [sel]
        else:
            nblk = (L + w.block_size - 1) // w.block_size
            pairs = []
            for i in range(nblk):
                blk = int(w.block_table[b, i])
                n = min(w.block_size, L - i * w.block_size)
                pairs.append((blk, slice(None), slice(0, n)))
        for sel in pairs:
            assert np.array_equal(kc[sel], ocache.k_codes[sel]), f"K codes differ (b={b}, {sel})"
            assert np.array_equal(vc[sel], ocache.v_codes[sel]), f"V codes differ (b={b}, {sel})"
            if ks is not None:
                assert ks[sel].tobytes() == ocache.k_scales[sel].tobytes(), f"K scales differ b={b}"
            if vs is not None:
                assert vs[sel].tobytes() == ocache.v_scales[sel].tobytes(), f"V scales differ b={b}"


def rel_errors(got: np.ndarray, ref: np.ndarray):
    num = np.linalg.norm((got - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    whole = num / den if den > 0 else num
    rows = got.reshape(-1, got.shape[-1]) - ref.reshape(-1, ref.shape[-1])
    rn = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    keep = rn > 0
    row = (np.linalg.norm(rows, axis=1)[keep] / rn[keep]).max() if keep.any() else 0.0
    zero_rows_ok = np.all(np.abs(rows[~keep]) == 0) if (~keep).any() else True
    return whole, row, zero_rows_ok


def check_output(got_bf16: torch.Tensor, ref: np.ndarray, what: str):
    got = got_bf16.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    whole, row, zok = rel_errors(got, ref)
    log(f"{what}: rel L2 {whole:.3e}, worst row {row:.3e}")
    assert zok, f"{what}: rows with zero reference output are not zero"
    assert whole <= REL_TOL, f"{what}: relative L2 error {whole:.3e} > {REL_TOL}"
    assert row <= ROW_TOL, f"{what}: worst row relative L2 {row:.3e} > {ROW_TOL}"
    return whole, row


def run_and_check(w: ki.Workload, what: str, max_seq_len=None, codes=True):
    t0 = time.time()
    cache = gpu_cache(w)
    table = gpu_build(w, cache)
    out = gpu_decode(w, cache, table, max_seq_len=max_seq_len)
    ref, _, ocache = oracle.reference(w)
    if codes:
        compare_codes(w, cache, ocache)
    res = check_output(out, ref, what)
    log(f"{what}: done in {time.time() - t0:.1f}s")
    return res
