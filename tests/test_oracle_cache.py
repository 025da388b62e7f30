"""Pins of the fp8 KV-cache write oracle (CPU only).

The encoder is checked against torch's own float8_e4m3fn conversion (a
library routine with the same definition: OCP e4m3fn, round to nearest even)
and against the format's code table; the quantiser against its defining
properties (the row maximum lands on +-448, the round-trip error is within
half a code step, zero rows)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encoder_matches_torch_on_random_values():
    rng = np.random.default_rng(11)
    # magnitudes across the whole range, including subnormals and ties
    x = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-12, 8.8, 200_000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    assert np.array_equal(oracle.e4m3fn_encode(x), _torch_codes(x))


def test_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.fp8_e4m3fn_to_f64(codes)
    back = oracle.e4m3fn_encode(vals)
    # +0 and -0 both decode to 0.0 with the sign kept by signbit
    assert np.array_equal(back, codes)


def test_encoder_ties_round_to_even():
    # midpoints between neighbouring codes: 1 + 1/16 lies between 1.0 (m=0)
    # and 1.125 (m=1): even mantissa wins; 1 + 3/16 -> 1.25 (m=2)
    x = np.array([1.0625, 1.1875, 2 ** -9 * 0.5, 2 ** -9 * 1.5, 448.0, -448.0], np.float32)
    got = oracle.e4m3fn_encode(x)
    assert got.tolist() == [0x38, 0x3A, 0x00, 0x02, 0x7E, 0xFE]


def test_quantiser_properties():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, 4, 128)) * np.exp2(rng.uniform(-4, 4, (64, 4, 1)))).astype(np.float32)
    x[3, 1] = 0.0                                   # an all-zero row
    codes, scale = oracle.quantize_token_heads(x)
    assert scale.dtype == np.float32 and scale[3, 1] == 1.0
    assert np.all(codes[3, 1] == 0)
    deq = oracle.fp8_e4m3fn_to_f64(codes) * scale[..., None]
    # the row maximum encodes to +-448 exactly
    amax_idx = np.argmax(np.abs(x), axis=-1)
    top = np.take_along_axis(np.abs(deq), amax_idx[..., None], -1)[..., 0]
    nz = scale != 1.0
    assert np.array_equal(top[nz], 448.0 * scale[nz].astype(np.float64))
    # every value within half a code step (relative 2^-4, absolute 2^-10 * scale)
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[..., None]) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_cache_write_places_tokens_and_skips_padding():
    rng = np.random.default_rng(13)
    N, Hkv, D, B, NB = 9, 2, 64, 16, 4
    k = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    slots = np.array([5, 17, -1, 63, 0, 32, -1, 48, 20])
    kc = np.full((NB, Hkv, B, D), 0x7F, np.uint8); vc = kc.copy()
    ks = np.full((NB, Hkv, B), np.nan, np.float32); vs = ks.copy()
    kc2, vc2, ks2, vs2 = oracle.cache_write_fp8(k, v, slots, kc, vc, ks, vs)
    kq, ksc = oracle.quantize_token_heads(k)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        assert np.array_equal(kc2[sl // B, :, sl % B], kq[t])
        assert np.array_equal(ks2[sl // B, :, sl % B], ksc[t])
    written = {int(s) for s in slots if s >= 0}
    for sl in range(NB * B):
        if sl not in written:
            assert np.all(kc2[sl // B, :, sl % B] == 0x7F) and np.all(np.isnan(ks2[sl // B, :, sl % B]))
