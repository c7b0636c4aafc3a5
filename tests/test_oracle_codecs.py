"""Pins for the oracle's codec decoders (no GPU).

Each decoder is written from the format definition; here it is compared, code
by code, with an independent library conversion or with integer enumeration.
"""
import numpy as np
import torch

import pytest

from oracle.codecs import (decode_bf16, decode_bit1, decode_fp8_e4m3, decode_fp16, decode_int4,
                           decode_int8, decode_uint2)
from synth.encode import encode_int_g32, pack_int4, pack_subbyte


def _same(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(both_nan | (a == b)))


def test_fp16_all_codes_match_numpy():
    codes = np.arange(1 << 16, dtype=np.uint16)
    assert _same(decode_fp16(codes), codes.view(np.float16).astype(np.float64))


def test_bf16_all_codes_match_torch():
    codes = np.arange(1 << 16, dtype=np.int32).astype(np.int16)
    ref = torch.from_numpy(codes).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(decode_bf16(codes.view(np.uint16)), ref)


def test_fp8_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_fp8_e4m3(codes)
    assert _same(got, ref)
    finite = got[np.isfinite(got)]
    assert finite.max() == 448.0 and finite.min() == -448.0
    assert np.min(np.abs(finite[finite != 0])) == 2.0 ** -9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.isfinite(got).sum() == 254          # no infinities, two NaN codes


def test_int8_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    assert np.array_equal(decode_int8(codes), codes.view(np.int8).astype(np.float64))


def test_int4_every_slot_and_value_brute_force():
    # element r of a word -> nibble slot, worked out by hand from the rule
    # "even elements in the low half-word, odd in the high half-word"
    slot = {0: 0, 1: 4, 2: 1, 3: 5, 4: 2, 5: 6, 6: 3, 7: 7}
    for r in range(8):
        for v in range(16):
            word = np.array([v << (4 * slot[r])], dtype="<u4").view(np.uint8)
            got = decode_int4(word[None, :])[0]
            expect = np.zeros(8)
            expect[r] = v - 16 if v >= 8 else v
            assert np.array_equal(got, expect)


def test_int_group_roundtrip_error_bound():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 64)).astype(np.float32) * 3
    for qmax, decode in ((127, None), (7, None)):
        codes, scales = encode_int_g32(x, qmax)
        s = scales.astype(np.float64).repeat(32, axis=-1)
        if qmax == 7:
            vals = decode_int4(pack_int4(codes)) * s
        else:
            vals = decode_int8(codes.view(np.uint8)) * s
        # Symmetric rounding: every element within half a step of its input,
        # up to the fp16 rounding of the scale (the largest element may sit
        # slightly past qmax*s and be clipped by at most qmax*|s - absmax/qmax|).
        amax = np.abs(x.reshape(5, 2, 32)).max(-1).repeat(32, -1)
        bound = s / 2 + np.abs(amax - qmax * s) + 1e-6
        assert np.all(np.abs(vals - x) <= bound)


def test_uint2_and_bit1_every_code():
    assert list(decode_uint2(np.arange(4))) == [0.0, 1.0, 2.0, 3.0]
    assert list(decode_bit1(np.array([0, 1]))) == [1.0, -1.0]
    with pytest.raises(ValueError):
        decode_uint2(np.array([4]))
    with pytest.raises(ValueError):
        decode_bit1(np.array([2]))


def test_subbyte_packing_hand_worked():
    """The generator's packing of 2- and 1-bit codes, against words worked
    out by hand from the rule: code r of a unit of m codes at slot
    (r % 2) * (m / 2) + r // 2."""
    def word(codes, bits):
        b = pack_subbyte(np.asarray(codes, np.uint8)[None], bits)[0]
        return int.from_bytes(b.tobytes(), "little")
    z16 = [0] * 16
    # INT2, 16 codes per 32-bit word: code 0 -> bits 0-1, code 1 -> slot 8
    # (bits 16-17), code 15 -> slot 15 (bits 30-31), code 6 -> slot 3 (bits 6-7)
    assert word([1] + z16[1:], 2) == 0x00000001
    assert word([0, 3] + z16[2:], 2) == 0x00030000
    assert word(z16[:15] + [2], 2) == 0x80000000
    assert word(z16[:6] + [3] + z16[7:], 2) == 0x000000C0
    # two words in a 32-code run: code 16 starts the second word
    assert word([0] * 16 + [1] + [0] * 15, 2) == 1 << 32
    # BIT1, 32 codes per word: code 1 -> bit 16, code 30 -> bit 15, code 31 -> bit 31
    z32 = [0] * 32
    assert word([0, 1] + z32[2:], 1) == 0x00010000
    assert word(z32[:30] + [1, 0], 1) == 0x00008000
    assert word(z32[:31] + [1], 1) == 0x80000000
    # BIT1 in a 2-byte run (head_dim 64): 16-bit unit, code 1 -> bit 8, code 15 -> bit 15
    assert word([0, 1] + z16[2:], 1) == 0x0100
    assert word(z16[:15] + [1], 1) == 0x8000
