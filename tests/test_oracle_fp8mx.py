"""Pins for the per-64-element tile quantiser (oracle.fp8.tile_exponent,
quantise_tiles, dequantise_tiles) and the "fp8mx" pool: the scale is the
smallest power of two that brings the tile into the E4M3 range (checked by
its defining inequality), codes equal torch's float8_e4m3fn conversion of the
scaled values, tokens are independent of their page neighbours, and decoding
is exact."""
import numpy as np
import torch

from oracle import fp8
from oracle import pool as op


def test_tile_exponent_is_the_smallest_fitting_power_of_two():
    rng = np.random.default_rng(0)
    vals = list(np.exp(rng.uniform(-60, 60, 4000)))
    vals += [448.0 * 2.0 ** k for k in range(-20, 21)]
    vals += [np.nextafter(448.0 * 2.0 ** k, np.inf) for k in range(-20, 21)]
    vals += [2.0 ** k for k in range(-40, 41)] + [1e-30, 3.3e30]
    for a in vals:
        a = float(np.float32(a))
        k = fp8.tile_exponent(a)
        assert a / 2.0 ** k <= 448.0, (a, k)
        assert a / 2.0 ** (k - 1) > 448.0, (a, k)
    assert fp8.tile_exponent(0.0) == 0


def test_tile_codes_match_torch_float8_and_decode_exactly():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((50, 3, 128)) * np.exp(rng.uniform(-8, 8, (50, 3, 1)))).astype(np.float32)
    x[0, 0, :64] = 0.0                              # an all-zero tile
    codes, exps = fp8.quantise_tiles(x)
    assert codes.shape == x.shape and exps.shape == (50, 3, 2)
    for i in range(50):
        for h in range(3):
            for g in range(2):
                t = x[i, h, 64 * g:64 * g + 64]
                k = int(exps[i, h, g]) - 127
                assert k == fp8.tile_exponent(np.max(np.abs(t)))
                y = torch.from_numpy(t) * (2.0 ** -k)
                want = torch.clamp(y, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                assert np.array_equal(codes[i, h, 64 * g:64 * g + 64], want)
    deq = fp8.dequantise_tiles(codes, exps)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = ref * np.repeat(2.0 ** (exps.astype(np.int64) - 127), 64, axis=-1)
    assert np.array_equal(deq, ref)
    # within half a step of the E4M3 grid (relative 2^-4) where not subnormal
    big = np.abs(x) >= np.repeat(np.max(np.abs(x.reshape(50, 3, 2, 64)), -1), 64, -1) * 2.0 ** -8
    assert np.all(np.abs(deq - x)[big] <= 2.0 ** -4 * np.abs(x)[big])


def test_fp8mx_pool_tokens_are_independent_of_page_neighbours():
    rng = np.random.default_rng(2)
    H, d = 2, 128
    k = (rng.standard_normal((40, H, d)) * 5).astype(np.float32)
    v = (rng.standard_normal((40, H, d)) * 0.1).astype(np.float32)
    a = op.PoolModel(8, 16, H, d, kv_dtype="fp8mx")
    b = op.PoolModel(8, 16, H, d, kv_dtype="fp8mx")
    a.alloc(0)
    b.alloc(0)
    a.append(0, k, v)
    for s in (slice(0, 7), slice(7, 16), slice(16, 40)):
        b.append(0, k[s], v[s])
    Ka, Va = a.gather(0)
    Kb, Vb = b.gather(0)
    assert np.array_equal(Ka, Kb) and np.array_equal(Va, Vb)
    kc, ke = fp8.quantise_tiles(k)
    assert np.array_equal(Ka, fp8.dequantise_tiles(kc, ke))
    # a path commit moves codes and scales unchanged
    a.commit_path(0, 12, [3, 7])
    K2, _ = a.gather(0)
    assert np.array_equal(K2[:29], Ka[:29]) and np.array_equal(K2[29], Ka[31]) and np.array_equal(K2[30], Ka[35])
