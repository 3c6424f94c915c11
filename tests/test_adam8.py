"""The hybrid 8-bit Adam with gradient clipping (LazyTrain abstract, on the
listing pages): the oracle's E4M3 format and block quantization pinned to a
library routine and to closed forms, the update pinned to the fp32 Adam,
and the host library's mt_host_adam8 bit for bit equal to the oracle."""
import ctypes as C

import numpy as np
import pytest

from oracle import adam8 as A8
from oracle import decoder as D


def _mt():
    from layer_streamed_amd import mt
    return mt


# ------------------------------------------------------------ oracle pins


def test_e4m3_values_match_torch_and_closed_form():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    mine = A8.e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))
    np.testing.assert_array_equal(mine[~np.isnan(mine)], ref[~np.isnan(ref)])
    # the format's landmarks: smallest subnormal, smallest normal, one, largest
    assert mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6
    assert mine[0x38] == 1.0 and mine[0x7E] == 448.0 and mine[0xB8] == -1.0
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])


def test_e4m3_encoding_matches_torch_rounding():
    """Round to nearest even against torch's float8_e4m3fn cast on values
    spread over the whole exponent range (in the format's finite range),
    exact midpoints between neighbours included."""
    import torch
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(400_000) * np.exp(rng.uniform(-14, 6.5, 400_000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    vals = A8.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)  # exact in fp32
    x = np.concatenate([x, mids, -mids, vals, np.float32([0.0, -0.0])])
    got = A8.e4m3_code(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)
    # every finite code round-trips; just above 448 saturates
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    np.testing.assert_array_equal(A8.e4m3_code(A8.e4m3_value(finite)), finite)
    assert A8.e4m3_code(np.float32([448.5, -470.0])).tolist() == [0x7E, 0xFE]


def test_block_quantization_error_bound():
    """Each block's largest magnitude maps to 448; a value whose scaled
    magnitude is normal (>= 2^-6) is within 2^-4 of itself (half a step of
    3 mantissa bits), a smaller one within 2^-10 of the scale."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(1000) * np.exp(rng.uniform(-8, 2, 1000))).astype(np.float32)
    x[256:384] = 0  # an all-zero block
    codes, scales = A8.quantize(x)
    assert scales.size == 8 and scales[2] == 0 and not codes[256:384].any()
    xh = A8.dequantize(codes, scales)
    for b, (lo, hi) in enumerate(A8.blocks(x.size)):
        blk, s = x[lo:hi], scales[b]
        if s == 0:
            continue
        assert np.isclose(s, np.abs(blk).max() / 448, rtol=1e-7)
        err = np.abs(xh[lo:hi] - blk)
        normal = np.abs(blk) / s >= 2.0 ** -6
        assert (err[normal] <= 2.0 ** -4 * np.abs(blk[normal]) * (1 + 1e-6)).all()
        assert (err[~normal] <= 2.0 ** -10 * s * (1 + 1e-6)).all()


def test_adam8_first_step_is_the_fp32_adam_and_states_within_bound():
    """From zero states the stored moments play no part: step 1 moves the
    master exactly as the fp32 Adam; the stored m and sqrt(v) then hold the
    fp32 Adam's moments within the quantization bound."""
    rng = np.random.default_rng(2)
    n = 1000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    hp = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)
    p8, st = A8.adam8_update(p, A8.zero_state(n), g, 1, **hp)
    p32, m32, v32 = D.adam_update(p, np.zeros_like(p), np.zeros_like(p), g, 1, **hp)
    np.testing.assert_array_equal(p8, p32)
    m8 = A8.dequantize(st[0], st[1])
    r8 = A8.dequantize(st[2], st[3])
    assert (np.abs(m8 - m32) <= 2.0 ** -4 * np.abs(m32) + 2.0 ** -10 * st[1].max()).all()
    assert (np.abs(r8 - np.sqrt(v32)) <= 2.0 ** -4 * np.sqrt(v32) + 2.0 ** -10 * st[3].max()).all()


def test_adam8_tracks_fp32_adam_over_steps():
    """Ten steps with fresh gradients: the 8-bit states move the weights
    within a few percent of the fp32 Adam's total movement."""
    rng = np.random.default_rng(3)
    n = 4096
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p8, st = p0.copy(), A8.zero_state(n)
    p32, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    for t in range(1, 11):
        g = (rng.standard_normal(n) * 1e-3 + 5e-4).astype(np.float32)
        p8, st = A8.adam8_update(p8, st, g, t, **hp)
        p32, m, v = D.adam_update(p32, m, v, g, t, **hp)
    d8, d32 = p8 - p0, p32 - p0
    assert np.linalg.norm(d8 - d32) / np.linalg.norm(d32) < 0.05


def test_clip_coefficient_closed_form():
    g = {"a": np.float32([3.0, 0.0]), "b": np.float32([[4.0]])}  # norm 5
    assert A8.clip_coefficient(g, 0.0) == 1.0
    assert A8.clip_coefficient(g, 10.0) == 1.0
    c = A8.clip_coefficient(g, 1.0)
    assert abs(c - 1.0 / (5.0 + 1e-6)) < 1e-7
    # the clipped gradient has norm max_norm (to the 1e-6 guard)
    tot = np.sqrt(sum(float(np.sum((x * c).astype(np.float64) ** 2)) for x in g.values()))
    assert abs(tot - 1.0) < 1e-6


# --------------------------------------------- host library against the oracle


def _lib_step(p, st, g, step, clip, dtype, shadow, threads, **hp):
    mt = _mt()
    cfg = mt.run_cfg(host_threads=threads, **hp)
    mc, ms, rc, rs = (a.copy() for a in st)
    sh = np.zeros(p.size, np.uint16) if shadow else None
    gbuf = D.bf16_bits(g) if dtype == mt.DT_BF16 else np.ascontiguousarray(g, np.float32)
    p = p.copy()
    status = mt.call("mt_host_adam8", mt.ptr(p), mt.ptr(mc), mt.ptr(ms), mt.ptr(rc), mt.ptr(rs),
                     mt.ptr(gbuf), dtype, mt.ptr(sh), p.size, step, clip, C.byref(cfg))
    return status, p, (mc, ms, rc, rs), sh


@pytest.mark.parametrize("dtype", [0, 1], ids=["bf16_grad", "f32_grad"])
@pytest.mark.parametrize("threads", [1, 7])
@pytest.mark.parametrize("shadow", [True, False], ids=["shadow", "no_shadow"])
def test_host_adam8_bitwise_equals_oracle(dtype, threads, shadow):
    mt = _mt()
    rng = np.random.default_rng(10 + dtype)
    n = 100_003  # a short last block
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    st_lib = st_or = A8.zero_state(n)
    p_lib = p_or = p
    hp = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)
    for step, clip in ((1, 1.0), (2, 0.37), (3, 1.0)):
        g = (rng.standard_normal(n) * np.exp(rng.uniform(-9, -3, n))).astype(np.float32)
        g[5000:5128] = 0  # a block with a zero gradient
        if dtype == mt.DT_BF16:
            g = D.bf16_round(g)
        status, p_lib, st_lib, sh = _lib_step(p_lib, st_lib, g, step, clip, dtype, shadow,
                                              threads, **hp)
        assert status == mt.MT_OK
        p_or, st_or = A8.adam8_update(p_or, st_or, g, step, clip=clip, **hp)
        np.testing.assert_array_equal(p_lib, p_or)
        for a, b in zip(st_lib, st_or):
            np.testing.assert_array_equal(a, b)
        if shadow:
            np.testing.assert_array_equal(sh, D.bf16_bits(p_or))


def test_host_adam8_validates_and_refuses_nonfinite():
    mt = _mt()
    n = 300
    p = np.ones(n, np.float32)
    st = A8.zero_state(n)
    g = np.ones(n, np.float32)
    g[17] = np.nan
    status, p2, st2, _ = _lib_step(p, st, g, 1, 1.0, mt.DT_F32, False, 2)
    assert status == mt.MT_E_NONFINITE
    np.testing.assert_array_equal(p2, p)
    for bad_clip in (0.0, 1.5):
        status, *_ = _lib_step(p, st, np.ones(n, np.float32), 1, bad_clip, mt.DT_F32, False, 2)
        assert status == mt.MT_E_INVALID
    status, *_ = _lib_step(p, st, np.ones(n, np.float32), 0, 1.0, mt.DT_F32, False, 2)
    assert status == mt.MT_E_INVALID


@pytest.mark.parametrize("simd", ["avx2", "scalar"])
def test_host_adam8_narrower_simd_paths_bitwise(simd):
    """The library takes the widest vector form the CPU has; MT_HOST_SIMD
    forces the narrower ones, which must give the same bits (the bitwise
    test above, in a fresh process with the variable set)."""
    import os
    import subprocess
    import sys
    env = dict(os.environ, MT_HOST_SIMD=simd)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-k",
                        "test_host_adam8_bitwise_equals_oracle", __file__],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "8 passed" in r.stdout, r.stdout[-500:]
