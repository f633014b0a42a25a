"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a hand-written
golden value, a format definition, a library routine (torch's fp8 cast, torch
SDPA), a closed form, an invariant the pages state, or brute force.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import kvq_inputs as ki
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
INT8, INT4, FP8, BF16 = 1, 2, 3, 4
PER_ROW, PER_TENSOR, PER_CHANNEL = 1, 2, 3


def _bits(t: torch.Tensor) -> np.ndarray:
    return ki.bf16_bits(t)


def _unpack_int4(codes: np.ndarray) -> np.ndarray:
    lo = (codes & 0xF).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    return np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)


SCALES = [1.0, 0.0301, 3.0 / 7.0, 2.0 ** -130, 2.0 ** 100, 1.0e-3]


# ------------------------------------------------------------- encoders

@pytest.mark.parametrize("dtype,qmax", [(INT8, 127), (INT4, 7)])
@pytest.mark.parametrize("scale", SCALES)
def test_int_encoder_every_bf16_value(oracle_lib, dtype, qmax, scale):
    """Every finite bf16 value: code == nearest integer of fp32(x / s) on [-Qmax, Qmax],
    ties to even (static scale, so the division is the only rounding before the code)."""
    bits, f = bf.all_finite_bf16()
    s = np.float32(scale)
    codes, _ = oracle_lib.quantize_rows(bits[None, :], dtype, PER_TENSOR, np.array([s]))
    got = codes[0].view(np.int8).astype(np.int64) if dtype == INT8 else _unpack_int4(codes)[0]
    with np.errstate(over="ignore"):
        y = (f / s).astype(np.float32)  # IEEE fp32 division, as the encoder's definition states
    want = bf.int_codes_argmin(y, qmax)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("scale", SCALES + [0.01004])
def test_fp8_encoder_every_bf16_value(oracle_lib, scale):
    bits, f = bf.all_finite_bf16()
    s = np.float32(scale)
    codes, _ = oracle_lib.quantize_rows(bits[None, :], FP8, PER_TENSOR, np.array([s]))
    with np.errstate(over="ignore"):
        y = (f / s).astype(np.float32)
    want = bf.fp8_codes_argmin(y)
    np.testing.assert_array_equal(codes[0].astype(np.int64), want)


# --------------------------------------------------- per-channel static scales
# "[CUDA] Add INT4 paged KV cache with per-channel scales", opening description
# and "Motivation and Context": static per-channel scales are per-(KV head,
# side) tables, element d of a row divided by its own channel's scale.

def _channel_table(D: int, seed: int) -> np.ndarray:
    """D distinct scales spanning 2^-20 .. 2^20, with 0, 2^-130 (subnormal),
    2^100, 1 and 3/7 among them."""
    rng = np.random.default_rng(seed)
    s = (2.0 ** rng.uniform(-20, 20, size=D)).astype(np.float32)
    s[[3, 17, 40, 41, 60]] = [0.0, 2.0 ** -130, 2.0 ** 100, 1.0, 3.0 / 7.0]
    assert len(np.unique(s)) == D
    return s


@pytest.mark.parametrize("dtype,qmax", [(INT8, 127), (INT4, 7), (FP8, 448)])
def test_per_channel_encoder_every_bf16_value(oracle_lib, dtype, qmax):
    """Every finite bf16 value quantized under a per-channel table: element d's code
    is the brute-force nearest code to fp32(x_d / s_d), 0 where s_d = 0.  The values
    are laid out in rows of D = 256 and rotated 4 times, so each value meets 4
    channels (4 different scales)."""
    bits, f = bf.all_finite_bf16()
    D = 256
    n = len(bits) // D * D
    table = _channel_table(D, 31 + dtype)
    for rot in (0, 1, 97, 200):
        rb = np.roll(bits[:n], rot).reshape(-1, D)
        rf = np.roll(f[:n], rot).reshape(-1, D)
        codes, scales = oracle_lib.quantize_rows(rb, dtype, PER_CHANNEL, table)
        assert not scales.any()  # a static mode writes no row scale
        with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
            y = (rf / table[None, :]).astype(np.float32)
        y = np.where(table[None, :] == 0, np.float32(0), y)
        if dtype == FP8:
            want = bf.fp8_codes_argmin(y.ravel()).reshape(y.shape)
            want = np.where(table[None, :] == 0, 0, want)  # s = 0 gives code 0x00
            got = codes.astype(np.int64)
        else:
            want = bf.int_codes_argmin(y.ravel(), qmax).reshape(y.shape)
            got = codes.view(np.int8).astype(np.int64) if dtype == INT8 else _unpack_int4(codes)
        np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("dtype,qmax", [(INT8, 127), (INT4, 7), (FP8, 448)])
@pytest.mark.parametrize("paged", [False, True])
def test_per_channel_append_and_dequantize_per_head(oracle_lib, dtype, qmax, paged):
    """Three KV heads with different per-channel tables (K and V tables differ
    too): every appended row's codes are the brute-force codes under its own
    head's table, and dequantize returns code x s[h, d] with the code read
    straight from the cache bytes."""
    Hkv, D, B, L = 3, 64, 2, 37
    rng = np.random.default_rng(90 + dtype + 10 * paged)
    kt = np.stack([_channel_table(D, 500 + h) for h in range(Hkv)]) * np.float32(0.01)
    vt = np.stack([_channel_table(D, 600 + h) for h in range(Hkv)]) * np.float32(0.02)
    kt, vt = kt.astype(np.float32), vt.astype(np.float32)
    # data of the size of each channel's scale, so codes spread over the grid
    k = torch.from_numpy((rng.standard_normal((B, L, Hkv, D)) * qmax / 3 * kt[None, None])
                         .astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy((rng.standard_normal((B, L, Hkv, D)) * qmax / 3 * vt[None, None])
                         .astype(np.float32)).to(torch.bfloat16)
    bs = 16 if paged else 48
    mb = (L + bs - 1) // bs if paged else 1
    nb = B * mb
    table = rng.permutation(nb).astype(np.int32).reshape(B, mb) if paged else None
    c = oracle_lib.Cache(dtype, PER_CHANNEL, Hkv, D, bs, nb, kt, vt)
    c.append(_bits(k), _bits(v), np.zeros(B, np.int32), table)
    lens = np.full(B, L, np.int32)
    Kd, Vd = c.dequantize(lens, table)
    kf, vf = k.float().numpy(), v.float().numpy()
    for b in range(B):
        for p in range(L):
            blk = b if table is None else table[b, p // bs]
            for h in range(Hkv):
                for side, x, tab, codes, deq in (("K", kf, kt, c.k_codes, Kd), ("V", vf, vt, c.v_codes, Vd)):
                    row = codes[blk, h, p % bs]
                    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
                        y = (x[b, p, h] / tab[h]).astype(np.float32)
                    y = np.where(tab[h] == 0, np.float32(0), y)
                    if dtype == FP8:
                        want = np.where(tab[h] == 0, 0, bf.fp8_codes_argmin(y))
                        got = row.astype(np.int64)
                        val = bf.fp8_value_table()[row]
                    else:
                        want = bf.int_codes_argmin(y, qmax)
                        got = row.view(np.int8).astype(np.int64) if dtype == INT8 else _unpack_int4(row[None])[0]
                        val = got.astype(np.float64)
                    np.testing.assert_array_equal(got, want, err_msg=f"{side} b={b} p={p} h={h}")
                    # x-hat = float(c) * s, one fp32 multiply
                    xh = (val.astype(np.float32) * tab[h]).astype(np.float32)
                    np.testing.assert_array_equal(deq[b, h, p], xh, err_msg=f"{side} dequant h={h}")


def test_fp8_encoder_matches_torch_cast_in_range(oracle_lib):
    """torch's float32 -> float8_e4m3fn cast (round to nearest even) agrees with the
    oracle wherever no saturation is involved."""
    bits, f = bf.all_finite_bf16()
    for s in (1.0, 0.0301, 2.0 ** -7):
        with np.errstate(over="ignore"):
            y = (f / np.float32(s)).astype(np.float32)
        y = y[np.abs(y) < 448.0]
        t = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = oracle_lib.fp8_encode(y[::7])
        np.testing.assert_array_equal(got, t[::7])


def test_fp8_decode_golden_and_torch(oracle_lib):
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "fp8_e4m3fn_points.txt"))
            if ln.strip() and not ln.startswith("#")]
    for code, val in rows:
        got = oracle_lib.lib().kvo_fp8_decode(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val), (code, got, val)
            assert math.copysign(1, got) == math.copysign(1, float(val))
    allc = np.arange(256, dtype=np.uint8)
    ours = oracle_lib.fp8_decode(allc)
    theirs = torch.from_numpy(allc).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    np.testing.assert_array_equal(ours[ok], theirs[ok])
    # every finite code re-encodes to itself (signed zero included)
    fin = allc[ok]
    np.testing.assert_array_equal(oracle_lib.fp8_encode(ours[ok].astype(np.float32)), fin)


def test_fp8_saturation_and_signed_zero(oracle_lib):
    y = np.array([448.0, 449.0, 463.9, 464.0, 1e30, -1e30, -0.0, 0.0, -1e-9, 2.0 ** -10,
                  3 * 2.0 ** -11, -(2.0 ** -10) * 1.0000001], np.float32)
    got = oracle_lib.fp8_encode(y)
    # 2^-10 is the midpoint of 0 and 2^-9: ties to the even code 0x00;
    # 3 * 2^-11 lies between 2^-10 and 2^-9, nearer 2^-9 (code 0x01).
    np.testing.assert_array_equal(got, [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80,
                                        0x00, 0x01, 0x81])


def test_int4_packing_golden(oracle_lib):
    for ln in open(os.path.join(GOLDEN, "int4_pack.txt")):
        if not ln.strip() or ln.startswith("#"):
            continue
        left, right = ln.split("->")
        codes = [int(c) for c in left.split()]
        want = bytes(int(b, 16) for b in right.split())
        # build a row whose codes are exactly `codes` at unit per-tensor scale
        x = torch.tensor(codes, dtype=torch.float32).to(torch.bfloat16)
        got, _ = oracle_lib.quantize_rows(_bits(x)[None, :], INT4, PER_TENSOR, np.array([1.0]))
        assert bytes(got[0]) == want


def test_zero_scale_and_zero_row(oracle_lib):
    x = torch.zeros(1, 64, dtype=torch.bfloat16)
    for dt in (INT8, INT4, FP8):
        codes, scales = oracle_lib.quantize_rows(_bits(x), dt, PER_ROW)
        assert scales[0] == 0.0 and not codes.any()
        xr = torch.randn(1, 64).to(torch.bfloat16)
        codes, _ = oracle_lib.quantize_rows(_bits(xr), dt, PER_TENSOR, np.array([0.0]))
        assert not codes.any()


# ------------------------------------------------- per-row quantization

@pytest.mark.parametrize("dtype,qmax", [(INT8, 127), (INT4, 7), (FP8, 448)])
def test_per_row_scale_is_absmax_over_qmax(oracle_lib, dtype, qmax):
    x = ki.randn_bf16((64, 256), 901)
    bits = _bits(x)
    codes, scales = oracle_lib.quantize_rows(bits, dtype, PER_ROW)
    xf = x.float().numpy()
    want = (np.abs(xf).max(axis=1).astype(np.float32) / np.float32(qmax)).astype(np.float32)
    np.testing.assert_array_equal(scales, want)
    if dtype != FP8:
        got = codes.view(np.int8).astype(np.int64) if dtype == INT8 else _unpack_int4(codes)
        # the absmax element always maps to +-Qmax
        idx = np.abs(xf).argmax(axis=1)
        assert np.all(np.abs(got[np.arange(64), idx]) == qmax)
        for i in range(64):
            y = (xf[i] / scales[i]).astype(np.float32)
            np.testing.assert_array_equal(got[i], bf.int_codes_argmin(y, qmax))
    else:
        for i in range(64):
            y = (xf[i] / scales[i]).astype(np.float32)
            np.testing.assert_array_equal(codes[i].astype(np.int64), bf.fp8_codes_argmin(y))


@pytest.mark.parametrize("dtype,qmax", [(INT8, 127), (INT4, 7)])
def test_round_trip_within_half_step(oracle_lib, dtype, qmax):
    """kv-quant-attn page, Correctness: appends round-trip within half a quantization step.

    Half a step exactly, plus the two fp32 roundings the definition contains: fl(x / s)
    moves y by at most |y| 2^-24 <= Qmax 2^-24 steps and fl(c * s) moves x-hat by at most
    Qmax s 2^-24, so |x - x-hat| <= s/2 (1 + 4 Qmax 2^-24)."""
    x = ki.randn_bf16((256, 256), 902)
    codes, scales = oracle_lib.quantize_rows(_bits(x), dtype, PER_ROW)
    xh = oracle_lib.dequantize_rows(codes, 256, dtype, PER_ROW, scales)
    err = np.abs(x.double().numpy() - xh.astype(np.float64))
    assert np.all(err <= scales[:, None].astype(np.float64) / 2 * (1 + 4 * qmax * 2.0 ** -24))


def test_dequantize_is_code_times_scale(oracle_lib):
    rng = np.random.default_rng(5)
    codes = rng.integers(-127, 128, size=(8, 64)).astype(np.int8).view(np.uint8)
    scales = rng.random(8).astype(np.float32)
    xh = oracle_lib.dequantize_rows(codes, 64, INT8, PER_ROW, scales)
    want = (codes.view(np.int8).astype(np.float32) * scales[:, None]).astype(np.float32)
    np.testing.assert_array_equal(xh, want)
    ch = rng.random(64).astype(np.float32)
    xh = oracle_lib.dequantize_rows(codes, 64, INT8, PER_CHANNEL, None, ch)
    np.testing.assert_array_equal(xh, (codes.view(np.int8).astype(np.float32) * ch).astype(np.float32))


# ------------------------------------------------------------- append

@pytest.mark.parametrize("dtype,mode", [(INT8, PER_ROW), (INT4, PER_ROW), (FP8, PER_TENSOR),
                                        (INT4, PER_CHANNEL), (FP8, PER_ROW)])
@pytest.mark.parametrize("paged", [False, True])
def test_bulk_append_equals_sequential_and_touches_nothing_else(oracle_lib, dtype, mode, paged):
    w = ki.random_workload(700 + dtype * 10 + mode, B=2, Hkv=2, G=2, D=64, Tq=1, lens=[40, 40],
                           dtype=dtype, mode=mode, block_size=16 if paged else None)
    kb, vb = _bits(w.k), _bits(w.v)
    mk = lambda: oracle_lib.Cache(w.dtype, w.mode, w.Hkv, w.D, w.block_size, w.num_blocks,
                                  w.k_static, w.v_static)
    bulk, seq = mk(), mk()
    for c in (bulk, seq):
        c.k_codes[...] = 0xA5
        c.v_codes[...] = 0x5A
        c.k_scales[...] = -7.0
        c.v_scales[...] = -9.0
    bt = w.block_table
    # contiguous: capacity 40 rows; write rows 3..39 in bulk vs one by one
    start = np.array([3, 3], np.int32)
    bulk.append(kb[:, 3:40], vb[:, 3:40], start, bt)
    for j in range(3, 40):
        seq.append(kb[:, j:j + 1], vb[:, j:j + 1], np.array([j, j], np.int32), bt)
    for a, b in [(bulk.k_codes, seq.k_codes), (bulk.v_codes, seq.v_codes),
                 (bulk.k_scales, seq.k_scales), (bulk.v_scales, seq.v_scales)]:
        assert a.tobytes() == b.tobytes()
    # rows 0..2 of every sequence, and every block no sequence maps, keep the fill
    written = np.zeros(bulk.k_codes.shape[:3], bool)
    for b in range(2):
        for p in range(3, 40):
            blk = b if bt is None else bt[b, p // w.block_size]
            written[blk, :, p % w.block_size] = True
    assert np.all(bulk.k_codes[~written] == 0xA5) and np.all(bulk.v_codes[~written] == 0x5A)
    if mode == PER_ROW:
        assert np.all(bulk.k_scales[~written] == -7.0) and np.all(bulk.v_scales[~written] == -9.0)
        assert np.all(bulk.k_scales[written] >= 0)
    else:
        assert np.all(bulk.k_scales == -7.0)  # static modes write no scale


# ------------------------------------------------------ unquantized bf16 cache
# kv-quant-attn page, "Performance": the int8 decode is compared with a bf16
# cache.  The same layout holds the bf16 values themselves and no scales.

def test_bf16_cache_stores_every_value_and_reads_it_back(oracle_lib):
    """Every bf16 bit pattern is stored as its own two bytes (little-endian)
    and read back as torch's bf16 -> fp32 conversion, bit for bit."""
    bits = np.arange(65536, dtype=np.uint16).reshape(256, 256)
    codes, scales = oracle_lib.quantize_rows(bits, BF16, 0)
    assert codes.shape == (256, 512)
    assert np.array_equal(codes.view("<u2"), bits)
    assert np.all(scales == 0)
    back = oracle_lib.dequantize_rows(codes, 256, BF16, 0)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(back.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("paged", [False, True])
def test_bf16_cache_append_writes_only_its_rows(oracle_lib, paged):
    w = ki.random_workload(760, B=2, Hkv=2, G=2, D=64, Tq=1, lens=[40, 40], dtype=BF16,
                           mode=PER_ROW, block_size=16 if paged else None)
    c = oracle_lib.Cache(w.dtype, w.mode, w.Hkv, w.D, w.block_size, w.num_blocks)
    assert c.mode == 0 and c.v_mode == 0 and c.k_codes.shape[-1] == 2 * w.D
    c.k_codes[...] = 0xA5
    c.v_codes[...] = 0x5A
    c.k_scales[...] = -7.0
    kb, vb = _bits(w.k), _bits(w.v)
    bt = w.block_table
    c.append(kb[:, 3:40], vb[:, 3:40], np.array([3, 3], np.int32), bt)
    written = np.zeros(c.k_codes.shape[:3], bool)
    for b in range(2):
        for p in range(3, 40):
            blk = b if bt is None else bt[b, p // w.block_size]
            written[blk, :, p % w.block_size] = True
            for h in range(2):
                row = c.k_codes[blk, h, p % w.block_size].view("<u2")
                assert np.array_equal(row, kb[b, p, h])
                assert np.array_equal(c.v_codes[blk, h, p % w.block_size].view("<u2"), vb[b, p, h])
    assert np.all(c.k_codes[~written] == 0xA5) and np.all(c.v_codes[~written] == 0x5A)
    assert np.all(c.k_scales == -7.0)  # no scales are written


@pytest.mark.parametrize("Tq,paged,sink", [(1, False, False), (3, True, True), (8, True, False)])
def test_bf16_cache_attention_matches_torch_sdpa(oracle_lib, Tq, paged, sink):
    """Decode over a bf16 cache is exact attention over the bf16 K and V values,
    with K and V taken from the workload by torch, not from the oracle cache."""
    w = ki.random_workload(770 + Tq, B=2, Hkv=2, G=3, D=64, Tq=Tq, lens=[Tq + 20, 75],
                           dtype=BF16, mode=PER_ROW, block_size=16 if paged else None,
                           sink=sink)
    out, lse, _ = oracle_lib.reference(w)
    K = w.k.float().permute(0, 2, 1, 3).contiguous().numpy()  # [B, Hkv, Lmax, D]
    V = w.v.float().permute(0, 2, 1, 3).contiguous().numpy()
    ref = _sdpa_ref(w.q.double().numpy(), K, V, w.lens, w.sm_scale, Tq)
    if sink:
        # o *= 1 / (1 + exp(s_h - lse)), with lse of the exact logits computed here
        G = w.Hq // w.Hkv
        qd = w.q.double()
        lse_ref = np.zeros((w.B, Tq, w.Hq))
        for b in range(w.B):
            L = int(w.lens[b])
            for j in range(Tq):
                for h in range(w.Hq):
                    z = float(w.sm_scale) * (torch.from_numpy(K[b, h // G, :L - Tq + j + 1]).double()
                                             @ qd[b, j, h])
                    lse_ref[b, j, h] = torch.logsumexp(z, 0).item()
        assert np.max(np.abs(lse - lse_ref)) <= 1e-12
        f = 1.0 / (1.0 + np.exp(w.sink.astype(np.float64)[None, None, :] - lse_ref))
        ref = ref * f[..., None]
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_sequential_build_of_tiny_workload(oracle_lib):
    """Workload 1 is built by 256 sequential one-row appends; a bulk build is identical."""
    w = ki.make_workload(1)
    c_bulk = oracle_lib.build_cache(w)
    c_seq = oracle_lib.Cache(w.dtype, w.mode, w.Hkv, w.D, w.block_size, w.num_blocks)
    kb, vb = _bits(w.k), _bits(w.v)
    for t in range(256):
        c_seq.append(kb[:, t:t + 1], vb[:, t:t + 1], np.array([t], np.int32))
    assert c_bulk.k_codes.tobytes() == c_seq.k_codes.tobytes()
    assert c_bulk.v_scales.tobytes() == c_seq.v_scales.tobytes()


# ------------------------------------------------------------ attention

def _sdpa_ref(q, K, V, lens, scale, Tq):
    """torch SDPA in float64 with GQA by repeat_interleave and an explicit causal mask."""
    B, _, Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for b in range(B):
        L = int(lens[b])
        qt = torch.from_numpy(q[b]).transpose(0, 1)  # [Hq, Tq, D]
        kt = torch.from_numpy(K[b, :, :L].astype(np.float64)).repeat_interleave(G, 0)
        vt = torch.from_numpy(V[b, :, :L].astype(np.float64)).repeat_interleave(G, 0)
        pos = L - Tq + torch.arange(Tq)[:, None]
        mask = torch.arange(L)[None, :] <= pos
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                             scale=float(scale))
        out[b] = o.transpose(0, 1).numpy()
    return out


@pytest.mark.parametrize("G,Tq", [(1, 1), (4, 1), (6, 3), (8, 8), (6, 37), (3, 90)])
def test_attend_matches_torch_sdpa_fp64(oracle_lib, G, Tq):
    """Causal attention of Tq query tokens ending at each sequence's length; the
    larger Tq are a chunked prefill (the chunk attends the cache and itself)."""
    rng = np.random.default_rng(G * 10 + Tq)
    B, Hkv, D = 2, 2, 64
    lens = np.array([max(37, Tq), 90], np.int32)
    K = rng.standard_normal((B, Hkv, 90, D)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, 90, D)).astype(np.float32)
    q = ki.randn_bf16((B, Tq, G * Hkv, D), 11 + G)
    scale = np.float32(1 / 8)
    out, _ = oracle_lib.attend(_bits(q), K, V, lens, scale)
    ref = _sdpa_ref(q.double().numpy(), K, V, lens, scale, Tq)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_attend_matches_python_loops_tiny(oracle_lib):
    for seed, (B, Hkv, G, D, Tq, lens) in enumerate([(1, 1, 2, 32, 1, [5]), (2, 2, 3, 32, 2, [1, 17]),
                                                     (1, 2, 4, 64, 3, [40]), (2, 1, 1, 32, 1, [3, 9])]):
        w = ki.random_workload(300 + seed, B=B, Hkv=Hkv, G=G, D=D, Tq=Tq, lens=lens, dtype=INT8,
                               mode=PER_ROW, sink=(seed % 2 == 1))
        out, _, cache = oracle_lib.reference(w)
        K, V = cache.dequantize(w.lens)
        ref = bf.attention_loops(w.q.double().numpy(), K, V, w.lens, w.sm_scale, w.sink)
        assert np.max(np.abs(out - ref)) <= 1e-12


# ------------------------------------------------- separate K and V scale modes
# ORT PR "[CUDA] PagedAttention: quantized KV cache ...": k_scale and v_scale are
# separate inputs; each side may use its own granularity.

@pytest.mark.parametrize("dtype", [INT8, INT4, FP8])
def test_mixed_modes_compose_the_pure_caches(oracle_lib, dtype):
    """A cache with K in mode A and V in mode B holds, byte for byte, the K side
    of an all-A cache and the V side of an all-B cache."""
    modes = (PER_ROW, PER_TENSOR, PER_CHANNEL)
    for km in modes:
        for vm in modes:
            if km == vm:
                continue
            w = ki.random_workload(800 + 10 * km + vm + dtype, B=2, Hkv=2, G=2, D=64, Tq=1,
                                   lens=[40, 19], dtype=dtype, mode=km, v_mode=vm, block_size=16)
            mixed = oracle_lib.build_cache(w)
            wk = ki.random_workload(800 + 10 * km + vm + dtype, B=2, Hkv=2, G=2, D=64, Tq=1,
                                    lens=[40, 19], dtype=dtype, mode=km, v_mode=km, block_size=16)
            wv = ki.random_workload(800 + 10 * km + vm + dtype, B=2, Hkv=2, G=2, D=64, Tq=1,
                                    lens=[40, 19], dtype=dtype, mode=vm, v_mode=vm, block_size=16)
            ck = oracle_lib.build_cache(wk)
            cv = oracle_lib.build_cache(wv)
            np.testing.assert_array_equal(mixed.k_codes, ck.k_codes)
            np.testing.assert_array_equal(mixed.v_codes, cv.v_codes)
            if km == PER_ROW:
                np.testing.assert_array_equal(mixed.k_scales, ck.k_scales)
            if vm == PER_ROW:
                np.testing.assert_array_equal(mixed.v_scales, cv.v_scales)
            K, V = mixed.dequantize(w.lens, w.block_table)
            K1, _ = ck.dequantize(w.lens, w.block_table)
            _, V1 = cv.dequantize(w.lens, w.block_table)
            np.testing.assert_array_equal(K, K1)
            np.testing.assert_array_equal(V, V1)


# ---------------------------------------------- soft cap and sliding window
# ORT PR "[CUDA] PagedAttention: quantized KV cache ...", "CUDA kernels": the
# paged decode kernel takes a softcap and a sliding window.

def test_softcap_window_match_python_loops_tiny(oracle_lib):
    cases = [(1, 1, 2, 32, 1, [9], 1.5, 0), (2, 2, 3, 32, 2, [1, 17], 0.0, 4),
             (1, 2, 4, 64, 3, [40], 2.0, 7), (2, 1, 1, 32, 4, [3, 9], 0.7, 2)]
    for seed, (B, Hkv, G, D, Tq, lens, cap, win) in enumerate(cases):
        w = ki.random_workload(700 + seed, B=B, Hkv=Hkv, G=G, D=D, Tq=Tq, lens=lens, dtype=INT8,
                               mode=PER_ROW, sink=(seed % 2 == 1), softcap=cap, window=win)
        out, _, cache = oracle_lib.reference(w)
        K, V = cache.dequantize(w.lens)
        # the cap is an fp32 argument, like the softmax scale
        ref = bf.attention_loops(w.q.double().numpy(), K, V, w.lens, w.sm_scale, w.sink,
                                 softcap=float(np.float32(cap)), window=win)
        assert np.max(np.abs(out - ref)) <= 1e-12


@pytest.mark.parametrize("window,Tq", [(1, 1), (5, 1), (16, 3), (33, 8)])
def test_window_matches_torch_sdpa_mask(oracle_lib, window, Tq):
    """The window as a boolean mask handed to torch SDPA in float64."""
    rng = np.random.default_rng(window * 10 + Tq)
    B, Hkv, G, D = 2, 2, 3, 64
    lens = np.array([37, 90], np.int32)
    K = rng.standard_normal((B, Hkv, 90, D)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, 90, D)).astype(np.float32)
    q = ki.randn_bf16((B, Tq, G * Hkv, D), 51 + window)
    scale = 1 / 8
    out, _ = oracle_lib.attend(_bits(q), K, V, lens, scale, window=window)
    for b in range(B):
        L = int(lens[b])
        qt = q[b].double().transpose(0, 1)
        kt = torch.from_numpy(K[b, :, :L].astype(np.float64)).repeat_interleave(G, 0)
        vt = torch.from_numpy(V[b, :, :L].astype(np.float64)).repeat_interleave(G, 0)
        pos = L - Tq + torch.arange(Tq)[:, None]
        t = torch.arange(L)[None, :]
        mask = (t <= pos) & (t > pos - window)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        assert np.max(np.abs(out[b] - ref.transpose(0, 1).numpy())) <= 1e-12


def test_window_and_softcap_limits(oracle_lib):
    rng = np.random.default_rng(77)
    B, Hkv, G, D, Tq, L = 1, 2, 2, 32, 3, 50
    K = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    q = ki.randn_bf16((B, Tq, G * Hkv, D), 78)
    lens = np.array([L], np.int32)
    base, _ = oracle_lib.attend(_bits(q), K, V, lens, 0.3)
    # a window covering the whole sequence changes nothing
    wide, _ = oracle_lib.attend(_bits(q), K, V, lens, 0.3, window=L)
    np.testing.assert_array_equal(wide, base)
    # window 1: each query sees only its own token, whose value row it returns
    one, _ = oracle_lib.attend(_bits(q), K, V, lens, 0.3, window=1)
    for j in range(Tq):
        for h in range(G * Hkv):
            np.testing.assert_array_equal(one[0, j, h], V[0, h // G, L - Tq + j].astype(np.float64))
    # an enormous cap is the identity on logits of size O(1)
    loose, _ = oracle_lib.attend(_bits(q), K, V, lens, 0.3, softcap=1e9)
    assert np.max(np.abs(loose - base)) <= 1e-12
    # a tiny cap flattens every logit to ~0: the mean of the visible value rows
    flat, _ = oracle_lib.attend(_bits(q), K, V, lens, 0.3, softcap=1e-9)
    for j in range(Tq):
        n = L - Tq + j + 1
        for h in range(G * Hkv):
            mean = V[0, h // G, :n].astype(np.float64).mean(axis=0)
            assert np.max(np.abs(flat[0, j, h] - mean)) <= 1e-7
    # the cap bounds the logit spread: weights stay within exp(2 c) of each other,
    # so a cap of 0.5 pulls the output towards the mean compared to no cap
    capped, _ = oracle_lib.attend(_bits(q), K, V, lens, 0.3, softcap=0.5)
    n = L - Tq + 1
    mean = V[0, 0, :n].astype(np.float64).mean(axis=0)
    assert np.linalg.norm(capped[0, 0, 0] - mean) < np.linalg.norm(base[0, 0, 0] - mean)


def test_gqa_matches_replicated_heads(oracle_lib):
    """kv-quant-attn page, Correctness: GQA ratios 1:1 .. 8:1 match a replicated-head reference."""
    rng = np.random.default_rng(8)
    for G in range(1, 9):
        B, Hkv, D, L = 1, 2, 32, 50
        K = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
        V = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
        q = ki.randn_bf16((B, 1, G * Hkv, D), 40 + G)
        lens = np.array([L], np.int32)
        out, _ = oracle_lib.attend(_bits(q), K, V, lens, 0.2)
        Kr = np.repeat(K, G, axis=1)
        Vr = np.repeat(V, G, axis=1)
        ref, _ = oracle_lib.attend(_bits(q), Kr, Vr, lens, 0.2)
        np.testing.assert_array_equal(out, ref)
        # and head h really reads KV head h // G
        one, _ = oracle_lib.attend(_bits(q[:, :, G:G + 1].contiguous()), K[:, 1:2], V[:, 1:2], lens, 0.2)
        np.testing.assert_array_equal(out[:, :, G], one[:, :, 0])


def test_head_sink_identity(oracle_lib):
    """The sink rescale 1/(1+exp(s - lse)) equals a softmax over [z, s] whose extra column
    carries a zero value vector; s -> -inf recovers plain attention."""
    rng = np.random.default_rng(9)
    B, Hkv, G, D, L = 1, 1, 3, 32, 30
    K = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    q = ki.randn_bf16((B, 1, G, D), 77)
    lens = np.array([L], np.int32)
    sink = np.array([0.5, -2.0, 3.0], np.float32)
    out, lse = oracle_lib.attend(_bits(q), K, V, lens, 0.25, sink)
    qd = q.double().numpy()
    for h in range(G):
        z = 0.25 * (K[0, 0].astype(np.float64) @ qd[0, 0, h])
        zz = np.concatenate([z, [float(sink[h])]])
        p = np.exp(zz - zz.max())
        p /= p.sum()
        ref = p[:L] @ V[0, 0].astype(np.float64)
        assert np.max(np.abs(out[0, 0, h] - ref)) <= 1e-13
    plain, _ = oracle_lib.attend(_bits(q), K, V, lens, 0.25)
    off, _ = oracle_lib.attend(_bits(q), K, V, lens, 0.25, np.full(3, -1e30, np.float32))
    np.testing.assert_array_equal(off, plain)


def test_max_logit_and_normalizer(oracle_lib):
    """The largest logit the oracle reports is the max of the fp64 logits computed
    here, and lse - m is the log of sum_t exp(z_t - m) (>= 0, 0 for one token)."""
    rng = np.random.default_rng(14)
    B, Hkv, G, D, L, Tq = 1, 2, 3, 32, 25, 2
    K = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    q = ki.randn_bf16((B, Tq, G * Hkv, D), 15)
    out, lse, m = oracle_lib.attend(_bits(q), K, V, np.array([L], np.int32), 0.3, window=7,
                                    return_max=True)
    qd = q.double().numpy()
    for j in range(Tq):
        pos = L - Tq + j
        for h in range(G * Hkv):
            # the softmax scale is an fp32 argument, widened
            z = float(np.float32(0.3)) * (K[0, h // G, pos - 6:pos + 1].astype(np.float64) @ qd[0, j, h])
            assert abs(m[0, j, h] - z.max()) <= 1e-13
            assert abs(lse[0, j, h] - (z.max() + math.log(np.exp(z - z.max()).sum()))) <= 1e-13
    _, lse1, m1 = oracle_lib.attend(_bits(q), K, V, np.array([1], np.int32), 0.3, return_max=True)
    assert np.all(np.isneginf(m1[0, 0])) and np.all(lse1[0, 1] == m1[0, 1])


def test_closed_forms(oracle_lib):
    rng = np.random.default_rng(10)
    D = 64
    V = rng.standard_normal((1, 1, 20, D)).astype(np.float32)
    K = rng.standard_normal((1, 1, 20, D)).astype(np.float32)
    q = ki.randn_bf16((1, 1, 2, D), 3)
    # one cached token: the output is that token's value row
    out, lse = oracle_lib.attend(_bits(q), K, V, np.array([1], np.int32), 0.125)
    np.testing.assert_array_equal(out[0, 0, 0], V[0, 0, 0].astype(np.float64))
    sink = np.array([0.3, -0.7], np.float32)
    outs, _ = oracle_lib.attend(_bits(q), K, V, np.array([1], np.int32), 0.125, sink)
    z0 = 0.125 * float(K[0, 0, 0].astype(np.float64) @ q.double().numpy()[0, 0, 1])
    want = V[0, 0, 0].astype(np.float64) / (1 + math.exp(float(sink[1]) - z0))
    assert np.max(np.abs(outs[0, 0, 1] - want)) <= 1e-14
    # identical key rows: uniform weights, the output is the mean value row
    Ks = np.repeat(K[:, :, :1], 20, axis=2)
    out, _ = oracle_lib.attend(_bits(q), Ks, V, np.array([20], np.int32), 0.125)
    assert np.max(np.abs(out[0, 0, 0] - V[0, 0].astype(np.float64).mean(0))) <= 1e-14
    # empty sequence: zeros
    out, lse = oracle_lib.attend(_bits(q), K, V, np.array([0], np.int32), 0.125, sink)
    assert not out.any() and np.all(np.isneginf(lse))


def test_large_channel_scale_zero_codes_is_finite(oracle_lib):
    """"[CUDA] Add INT4 paged KV cache ...": q = 100 with a per-channel K scale of 1000 over
    all-zero K codes used to give NaN through an fp16 fold.  The exact answer is uniform
    attention: the mean of the dequantized value rows."""
    D, L = 256, 33
    w = ki.random_workload(55, B=1, Hkv=1, G=2, D=D, Tq=1, lens=[L], dtype=INT4, mode=PER_CHANNEL)
    w.q = torch.full_like(w.q, 100.0)
    w.k = torch.zeros_like(w.k)
    w.k_static = np.full((1, D), 1000.0, np.float32)
    out, _, cache = oracle_lib.reference(w)
    assert not cache.k_codes.any()
    _, V = cache.dequantize(w.lens)
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out[0, 0, 0] - V[0, 0].astype(np.float64).mean(0))) <= 1e-13


def test_causal_drafts(oracle_lib):
    """Query j of Tq sees exactly tokens t <= len - Tq + j (drafts are causal)."""
    rng = np.random.default_rng(12)
    D, L, Tq = 32, 24, 4
    K = rng.standard_normal((1, 1, L, D)).astype(np.float32)
    V = rng.standard_normal((1, 1, L, D)).astype(np.float32)
    q = ki.randn_bf16((1, Tq, 1, D), 12)
    out, _ = oracle_lib.attend(_bits(q), K, V, np.array([L], np.int32), 0.3)
    for j in range(Tq):
        n = L - Tq + j + 1
        one, _ = oracle_lib.attend(_bits(q[:, j:j + 1].contiguous()), K[:, :, :n], V[:, :, :n],
                                   np.array([n], np.int32), 0.3)
        np.testing.assert_array_equal(out[:, j], one[:, 0])


# ----------------------------------------------------- quality band, footprint

def test_quantization_error_band(oracle_lib):
    """kv-quant-attn page, Correctness: int8 ~1.0e-2 relative (cos 0.99995), int4 ~1.8e-1
    (cos 0.984) against unquantized attention, per-row absmax, Hq24 Hkv4 D256.  Accept +-25 %."""
    band = {ln.split()[0]: (float(ln.split()[1]), float(ln.split()[2]))
            for ln in open(os.path.join(GOLDEN, "quality_band.txt")) if ln[0] != "#"}
    for name, dt in (("int8", INT8), ("int4", INT4)):
        w = ki.make_workload(3, ctx=4096, dtype=name)
        out, _, _ = oracle_lib.reference(w)
        Kf = w.k.float().numpy().transpose(0, 2, 1, 3).copy()
        Vf = w.v.float().numpy().transpose(0, 2, 1, 3).copy()
        exact, _ = oracle_lib.attend(_bits(w.q), Kf, Vf, w.lens, w.sm_scale)
        rel = np.linalg.norm(out - exact) / np.linalg.norm(exact)
        cos = np.sum(out * exact) / (np.linalg.norm(out) * np.linalg.norm(exact))
        want_rel, want_cos = band[name]
        assert 0.75 * want_rel <= rel <= 1.25 * want_rel, (name, rel)
        assert abs((1 - cos) - (1 - want_cos)) <= 0.5 * (1 - want_cos), (name, cos)


def test_footprint(oracle_lib):
    for ln in open(os.path.join(GOLDEN, "footprint.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        bits, prs, layers, hkv, d, tokens, want = (int(x) for x in ln.split())
        got = oracle_lib.cache_bytes_per_token(bits, bool(prs), layers, hkv, d) * tokens
        assert got == want


def test_inputs_are_seeded():
    a = ki.make_workload(4, max_len=300)
    b = ki.make_workload(4, max_len=300)
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and np.array_equal(a.lens, b.lens)
    assert np.array_equal(a.block_table, b.block_table)
    assert sorted(a.block_table.ravel().tolist()) == list(range(a.num_blocks))
