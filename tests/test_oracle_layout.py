"""Pins for the oracle's in-page layout reader (no GPU).

Single codes are placed by hand at byte positions worked out on paper from
the layout definition; the reader must find each at the right (token, dim).
Then the generator's writer and the oracle's reader (two separate
implementations of the definition) must agree on random pages of every codec.
"""
import numpy as np
import pytest
import torch

from oracle.layout import code_bits, code_position, plane_values
from synth.encode import encode_affine2_g32, encode_int_g32, encode_sign1_g32
from synth.layout import BF16, BIT1, FP8, FP16, INT2, INT4, INT8, encode_plane


def test_code_position_hand_worked():
    # FP8, P=32, D=32: tile 512 B, run R = 8 B (no chunk interleave).
    k, _ = code_position(32, 32, FP8, is_v=False)
    # K (5, 7): kq = 7 // 8 = 0, e = 7 -> lane 5 -> 8*5 + 7 = 47
    assert k[5, 7] == 47
    # K (21, 19): tile 1, kq = 2, e = 3 -> lane 37 -> 512 + 8*37 + 3 = 811
    assert k[21, 19] == 811
    v, _ = code_position(32, 32, FP8, is_v=True)
    # V (5, 7): qd 1, j 1, c 7 -> lane 23, e = 1 -> 8*23 + 1 = 185
    assert v[5, 7] == 185
    # V (21, 19): tile 1, qd 1, j 1, n 1, c 3 -> lane 19, e = 5 -> 512 + 152 + 5 = 669
    assert v[21, 19] == 669
    for pos in (k, v):
        assert np.array_equal(np.sort(pos.ravel()), np.arange(32 * 32))
    # FP8, D=128: run 32 B, two 16-byte chunks interleaved over the 64 lanes.
    k, _ = code_position(16, 128, FP8, is_v=False)
    # (3, 100): kq 3, e 4 -> lane 51, chunk 0 -> 16*51 + 4 = 820
    assert k[3, 100] == 820
    # (3, 121): kq 3, e 25 -> lane 51, chunk 1 -> 1024 + 816 + 9 = 1849
    assert k[3, 121] == 1849
    assert np.array_equal(np.sort(k.ravel()), np.arange(16 * 128))
    # FP16 V, D=128: run 64 B. (6, 37): qd 1, j 2, c 5, n 2 -> lane 21,
    # e = 10 -> run byte 20 -> chunk 1 -> 1024 + 16*21 + 4 = 1364
    v, _ = code_position(16, 128, FP16, is_v=True)
    assert v[6, 37] == 1364
    # INT8 K (group scales), D=64: run 16 B. (2, 45): c 1, kq 1, j 5 ->
    # lane 18, e = 13 -> 16*18 + 13 = 301
    k, _ = code_position(16, 64, INT8, is_v=False)
    assert k[2, 45] == 301
    # INT4 K, D=32: run 4 B. (3, 5): lane 3, e 5 -> nibble slot 6 -> byte
    # 4*3 + 3 = 15, low nibble
    k, nib = code_position(16, 32, INT4, is_v=False)
    assert k[3, 5] == 15 and nib[3, 5] == 0


def test_code_bits_hand_worked():
    # INT2 K, P=16, D=128: run 8 B, 32-bit units of 16 codes. (3, 37): group
    # 1, kq 0, j 5 -> lane 3, e = 13 -> slot (1)*8 + 6 = 14 -> bit 28 ->
    # byte 3, bit 4 -> offset 8*3 + 3 = 27
    k, sh = code_bits(16, 128, INT2, is_v=False)
    assert k[3, 37] == 27 and sh[3, 37] == 4
    # BIT1 V, P=16, D=64: run 2 B, one 16-bit unit. (5, 20): qd 1, j 1,
    # n 1, c 4 -> lane 20, e = 5 -> slot 8 + 2 = 10 -> byte 1, bit 2 ->
    # offset 2*20 + 1 = 41
    v, sh = code_bits(16, 64, BIT1, is_v=True)
    assert v[5, 20] == 41 and sh[5, 20] == 2
    # every code owns its own bits, and together they fill the head's bytes
    for codec, bits in ((INT2, 2), (BIT1, 1), (INT4, 4)):
        for D in (64, 128):
            for is_v in (False, True):
                off, sh = code_bits(32, D, codec, is_v)
                at = np.sort((off * 8 + sh).ravel())
                assert np.array_equal(at, np.arange(32 * D) * bits)


def test_single_int2_code_scale_and_offset():
    hkv, P, D = 1, 16, 64
    codes = P * D // 4
    gb = P * (D // 32) * 2
    pool = np.zeros(codes + 2 * gb, dtype=np.uint8)
    # K (3, 5): lane 3, e 5 -> slot 8 + 2 = 10 -> bit 20 -> byte 4*3 + 2, bit 4; code 3
    pool[14] = 3 << 4
    # token 3, group 0: scale 0.5 at codes + 3*2*2, offset -1 at codes + gb + 12
    pool[codes + 12:codes + 14] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    pool[codes + gb + 12:codes + gb + 14] = np.frombuffer(np.float16(-1.0).tobytes(), np.uint8)
    k = plane_values(pool, 0, INT2, hkv, P, D, 0, 1.0, False, P)
    want = np.zeros((P, D))
    want[3, :32] = -1.0                                # code 0: the offset
    want[3, 5] = -1.0 + 0.5 * 3
    assert np.array_equal(k, want)


def test_single_bit1_code_and_scale():
    hkv, P, D = 1, 16, 64
    codes = P * D // 8
    pool = np.zeros(codes + P * (D // 32) * 2, dtype=np.uint8)
    pool[41] = 1 << 2                                  # V (5, 20): negative
    pool[codes + 20:codes + 22] = np.frombuffer(np.float16(0.25).tobytes(), np.uint8)  # token 5, group 0
    v = plane_values(pool, 0, BIT1, hkv, P, D, 0, 1.0, True, P)
    want = np.zeros((P, D))
    want[5, :32] = 0.25
    want[5, 20] = -0.25
    assert np.array_equal(v, want)


def test_single_fp16_code_in_k_and_v():
    hkv, P, D = 2, 32, 32
    pool = np.zeros(hkv * P * D * 2, dtype=np.uint8)
    head = 1
    # V (21, 19) of head 1: tile 1 (1024 B each), lane 19, e = 5 -> byte 1338
    pos = head * P * D * 2 + 1338
    pool[pos:pos + 2] = np.frombuffer(np.float16(1.5).tobytes(), np.uint8)
    v = plane_values(pool, 0, FP16, hkv, P, D, head, 1.0, True, P)
    assert v[21, 19] == 1.5 and np.count_nonzero(v) == 1
    # the same bytes read as K: lane 19 = 16*1 + 3 -> token 19, dim 8 + 5
    k = plane_values(pool, 0, FP16, hkv, P, D, head, 1.0, False, P)
    assert k[19, 13] == 1.5 and np.count_nonzero(k) == 1


def test_single_int4_code_and_scale():
    hkv, P, D = 1, 16, 32
    codes = P * D // 2
    pool = np.zeros(codes + P * (D // 32) * 2, dtype=np.uint8)
    # K element (3, 5) -> byte 15, low nibble; value -3 -> 0xD
    pool[15] = 0x0D
    # scale of token 3, group 0 -> fp16 at codes + 3*2
    pool[codes + 6:codes + 8] = np.frombuffer(np.float16(0.25).tobytes(), np.uint8)
    k = plane_values(pool, 0, INT4, hkv, P, D, 0, 1.0, False, P)
    assert k[3, 5] == -0.75 and np.count_nonzero(k) == 1


def test_fp8_scale_applied():
    hkv, P, D = 1, 16, 16
    pool = np.zeros(P * D, dtype=np.uint8)
    pool[0] = 0x38                                     # e=7, m=0 -> 1.0
    k = plane_values(pool, 0, FP8, hkv, P, D, 0, 0.5, False, P)
    assert k[0, 0] == 0.5


@pytest.mark.parametrize("codec", [FP16, BF16, FP8, INT8, INT4, INT2, BIT1])
@pytest.mark.parametrize("is_v", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_writer_reader_agree(codec, is_v, D):
    rng = np.random.default_rng(3)
    hkv, P = 2, 32
    x = rng.standard_normal((1, hkv, P, D)).astype(np.float32)
    plane, fp8s = encode_plane(x, codec, v_order=is_v)
    for h in range(hkv):
        got = plane_values(plane[0], 0, codec, hkv, P, D, h, fp8s[0, h], is_v, P)
        xh = x[0, h]
        if codec == FP16:
            ref = xh.astype(np.float16).astype(np.float64)
        elif codec == BF16:
            ref = torch.from_numpy(xh).to(torch.bfloat16).to(torch.float64).numpy()
        elif codec == FP8:
            s = np.float32(fp8s[0, h])
            c = torch.from_numpy(np.clip(xh / s, -448, 448)).to(torch.float8_e4m3fn)
            ref = c.to(torch.float64).numpy() * float(s)
        elif codec == INT2:
            u, sc, z = encode_affine2_g32(xh)
            ref = z.astype(np.float64).repeat(32, axis=-1) + u * sc.astype(np.float64).repeat(32, axis=-1)
        elif codec == BIT1:
            b, sc = encode_sign1_g32(xh)
            ref = np.where(b == 1, -1.0, 1.0) * sc.astype(np.float64).repeat(32, axis=-1)
        else:
            cq, sc = encode_int_g32(xh, 127 if codec == INT8 else 7)
            ref = cq.astype(np.float64) * sc.astype(np.float64).repeat(32, axis=-1)
        assert np.array_equal(got, ref)
