"""Pins for the oracle's in-page layout reader (no GPU).

Single codes are placed by hand at byte positions worked out on paper from
the layout definition; the reader must find each at the right (token, dim).
Then the generator's writer and the oracle's reader (two separate
implementations of the definition) must agree on random pages of every codec.
"""
import numpy as np
import pytest
import torch

from oracle.layout import element_index, plane_values
from synth.encode import encode_int_g32
from synth.layout import BF16, FP8, FP16, INT4, INT8, encode_plane


def test_element_index_hand_worked():
    # P=32, D=32. K: (t, i) -> t*32 + i.
    k = element_index(32, 32, is_v=False)
    assert k[5, 7] == 167 and k[31, 31] == 1023
    v = element_index(32, 32, is_v=True)
    # (t=5, i=7): tile 0, quad 1, token-in-quad 1, dim block 0, dim-in-block 7
    #   -> ((1*16 + 7) * 2 + 0) * 4 + 1 = 185
    assert v[5, 7] == 185
    # (t=21, i=19): tile 1 (base 512), quad 1, j 1, block 1, c 3
    #   -> 512 + ((16 + 3) * 2 + 1) * 4 + 1 = 669
    assert v[21, 19] == 669
    # (t=0, i=16): block 1 of lane (0, 0) -> 4
    assert v[0, 16] == 4
    # every position used exactly once
    assert np.array_equal(np.sort(v.ravel()), np.arange(32 * 32))


def test_single_fp16_code_in_k_and_v():
    hkv, P, D = 2, 32, 32
    pool = np.zeros(hkv * P * D * 2, dtype=np.uint8)
    head = 1
    pos = head * P * D * 2 + 669 * 2                  # V element (21, 19) of head 1
    pool[pos:pos + 2] = np.frombuffer(np.float16(1.5).tobytes(), np.uint8)
    v = plane_values(pool, 0, FP16, hkv, P, D, head, 1.0, True, P)
    assert v[21, 19] == 1.5 and np.count_nonzero(v) == 1
    k = plane_values(pool, 0, FP16, hkv, P, D, head, 1.0, False, P)
    t, i = divmod(669, D)
    assert k[t, i] == 1.5 and np.count_nonzero(k) == 1


def test_single_int4_code_and_scale():
    hkv, P, D = 1, 16, 32
    codes = P * D // 2
    pool = np.zeros(codes + P * (D // 32) * 2, dtype=np.uint8)
    # K element (3, 5) -> element 101 -> word 12, r = 5 -> nibble slot 6
    # (bits 24..27) -> byte 48 + 3 = 51, low nibble; value -3 -> 0xD
    pool[51] = 0x0D
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


@pytest.mark.parametrize("codec", [FP16, BF16, FP8, INT8, INT4])
@pytest.mark.parametrize("is_v", [False, True])
def test_writer_reader_agree(codec, is_v):
    rng = np.random.default_rng(3)
    hkv, P, D = 2, 32, 64
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
        else:
            cq, sc = encode_int_g32(xh, 127 if codec == INT8 else 7)
            ref = cq.astype(np.float64) * sc.astype(np.float64).repeat(32, axis=-1)
        assert np.array_equal(got, ref)
