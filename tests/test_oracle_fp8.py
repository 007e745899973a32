"""Pins for the oracle's E4M3 decoder."""
import math

import numpy as np
import torch

from oracle import fp8


def test_hand_derived_codes():
    # (code, value) from the encoding: sign | exponent (bias 7) | 3-bit mantissa
    cases = [
        (0x00, 0.0), (0x80, -0.0),
        (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),          # subnormals m * 2^-9
        (0x08, 2.0 ** -6),                                 # smallest normal
        (0x38, 1.0), (0xB8, -1.0), (0x39, 1.125), (0x3C, 1.5),
        (0x40, 2.0), (0x48, 4.0), (0x50, 8.0),
        (0x77, 240.0), (0x7E, 448.0), (0xFE, -448.0),      # largest finite
    ]
    got = fp8.decode_e4m3([c for c, _ in cases])
    for (code, want), g in zip(cases, got):
        assert g == want and math.copysign(1, g) == math.copysign(1, want), (hex(code), g, want)
    assert np.isnan(fp8.decode_e4m3([0x7F, 0xFF])).all()


def test_matches_torch_float8_e4m3fn_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.decode_e4m3(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), codes[~same]


def test_every_finite_code_is_exact_in_fp16():
    vals = fp8.decode_e4m3(np.arange(256, dtype=np.uint8))
    fin = np.isfinite(vals)
    assert np.array_equal(vals[fin].astype(np.float16).astype(np.float64), vals[fin])


def test_decode_pool_uses_the_same_table():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 256, size=(3, 5, 7), dtype=np.uint8)
    a = fp8.decode_pool(codes)
    b = fp8.decode_e4m3(codes.ravel()).reshape(codes.shape)
    assert np.array_equal(np.nan_to_num(a, nan=7.0), np.nan_to_num(b, nan=7.0))


def test_e4m3_decode_step_equals_fp16_pool_of_the_decoded_values():
    """The E4M3 path differs from the fp16 path only in how stored elements
    become values: a pool of codes and an fp16 pool holding their exact
    values give bit-identical oracle results."""
    import workload as W
    from oracle import attention as OA
    wl = W.custom("f8", 2, [37, 100], seed=3, kv_format="e4m3")
    m = W.materialise(wl, "cpu")
    assert m.pool.dtype == torch.uint8
    q = W.make_query(m, 0).numpy()
    codes = m.pool.numpy()
    vals16 = fp8.decode_pool(codes).astype(np.float16)
    o8, m8 = OA.decode_step(q, codes, m.table_host, m.lens, 0.0883883, kv_format="e4m3")
    o16, m16 = OA.decode_step(q, vals16, m.table_host, m.lens, 0.0883883)
    assert np.array_equal(o8, o16)
    for a, b in zip(m8, m16):
        assert np.array_equal(a, b)
    # spare blocks hold the NaN code
    used = np.zeros(m.pool_blocks, bool)
    used[m.table_host[m.table_host >= 0]] = True
    assert (codes[~used] == 0x7F).all()
