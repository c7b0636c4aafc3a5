"""Pins for oracle/encode.py (page encode / demotion and token append).

Checked against things other than the oracle itself: torch's float8_e4m3fn
cast (round to nearest even) on every e4m3 value and every midpoint, closed
forms (the absmax element maps to the largest code, all-zero blocks), error
bounds of the round trip, and the input generator's encoders (synth/), an
independent implementation of the same definitions and of the in-page layout.
"""
import numpy as np
import pytest
import torch

from oracle import codecs
from oracle.encode import (append_token, encode_block_fp8, encode_groups_affine2, encode_groups_int,
                           encode_groups_sign1, encode_page, fp32_to_e4m3)
from oracle.layout import BF16, BIT1, FP8, FP16, INT2, INT4, INT8, plane_values
from synth import encode as senc
from synth import layout as slay

E4M3 = codecs.decode_fp8_e4m3(np.arange(256))


def torch_e4m3(y):
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_exact_values_map_to_themselves():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = E4M3[codes].astype(np.float32)
    got = fp32_to_e4m3(vals)
    assert np.array_equal(got, codes)


def test_e4m3_midpoints_round_to_even_like_torch():
    pos = np.sort(E4M3[:0x7F])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)   # midpoints exact in fp32
    for sign in (1, -1):
        y = sign * mids
        assert np.array_equal(fp32_to_e4m3(y), torch_e4m3(y))
    # the tie goes to the even code
    got = fp32_to_e4m3(mids)
    assert np.all(got % 2 == 0)


def test_e4m3_random_and_signs_like_torch():
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-0.02, 0.02, 20000),
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -9 * 1.5]]).astype(np.float32)
    assert np.array_equal(fp32_to_e4m3(y), torch_e4m3(y))
    assert fp32_to_e4m3(np.float32(-0.0)) == 0x80
    with pytest.raises(ValueError):
        fp32_to_e4m3(np.float32(449.0))


def test_fp8_block_closed_forms_and_bound():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)).astype(np.float16).astype(np.float32)
    codes, s = encode_block_fp8(x)
    amax = np.max(np.abs(x))
    assert s == np.float32(amax / np.float32(448.0))
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] == (0x7E if x[i] > 0 else 0xFE)                  # +-448
    y = E4M3[codes] * np.float64(s)
    err = np.abs(y - x)
    # half an e4m3 step: 2^-4 relative for normals, 2^-10 absolute (times s) below 2^-6
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6)
    assert np.all(err <= bound)
    z, sz = encode_block_fp8(np.zeros((16, 64), np.float32))
    assert sz == 1.0 and not z.any()


@pytest.mark.parametrize("qmax", [127, 7])
def test_int_groups_closed_forms_and_bound(qmax):
    rng = np.random.default_rng(qmax)
    x = (rng.standard_normal((16, 128)) * rng.uniform(0.1, 10, (16, 1))).astype(np.float16).astype(np.float32)
    x[3, 32:64] = 0.0                                                 # one all-zero group
    codes, s = encode_groups_int(x, qmax)
    g = x.reshape(16, 4, 32)
    amax = np.abs(g).max(-1)
    assert np.array_equal(s[amax > 0], (amax[amax > 0] / np.float32(qmax)).astype(np.float16))
    assert s[3, 1] == 1.0 and not codes[3, 32:64].any()
    c = codes.reshape(16, 4, 32).astype(np.float64)
    idx = np.abs(g).argmax(-1)
    top = np.take_along_axis(c, idx[..., None], -1)[..., 0]
    ok = amax > 0
    assert np.all(np.abs(top[ok]) == qmax)                           # absmax element -> +-qmax
    s64 = s.astype(np.float64)[..., None]
    err = np.abs(c * s64 - g)
    excess = np.maximum(0, amax - qmax * s.astype(np.float64))[..., None]
    assert np.all(err <= s64 / 2 + excess + 1e-12)
    assert np.all(np.abs(codes) <= qmax)


@pytest.mark.parametrize("qmax", [127, 7])
def test_int_scale_stays_inside_fp16_range(qmax):
    """A group whose absmax / qmax rounds to 0 in fp16 gets the smallest
    positive fp16 scale 2^-24 (codes x / 2^-24, exact here); one whose scale
    overflows gets 65504 and saturated codes."""
    x = np.zeros((2, 64), np.float32)
    x[0, :32] = np.float32(2.0 ** -24) * np.array([1, -1] * 16, np.float32)   # fp16 min subnormal
    x[0, 32:] = np.float32(2.0 ** -23)
    x[1, :32] = np.float32(1e30) * np.array([1, -1] * 16, np.float32)          # a BF16-range group
    x[1, 32:] = np.float32(1e6)
    codes, s = encode_groups_int(x, qmax)
    assert s[0, 0] == np.float16(2.0 ** -24) and s[0, 1] == np.float16(2.0 ** -24)
    assert np.array_equal(codes[0, :32], np.array([1, -1] * 16)) and np.all(codes[0, 32:] == 2)
    assert s[1, 0] == np.float16(65504.0) and np.array_equal(codes[1, :32], np.array([qmax, -qmax] * 16))
    want = np.float16(min(1e6 / qmax, 65504.0))
    assert s[1, 1] == want and np.all(np.isfinite(codes.astype(np.float64)))
    c_gen, s_gen = senc.encode_int_g32(x, qmax)
    assert np.array_equal(codes, c_gen) and np.array_equal(s, s_gen)


def test_int_ties_go_to_the_even_code():
    """Quotients exactly halfway between two codes take the even one (rint,
    ties to even), for both signs and both widths. The group's absmax is
    qmax, so its scale is exactly 1 and each value is its own quotient; the
    expected codes are written out by hand."""
    # INT8 (qmax 127): value -> code
    int8 = {0.5: 0, 1.5: 2, 2.5: 2, 3.5: 4, 64.5: 64, 65.5: 66, 125.5: 126, 126.5: 126,
            -0.5: 0, -1.5: -2, -2.5: -2, -3.5: -4, -64.5: -64, -65.5: -66, -125.5: -126, -126.5: -126}
    # INT4 (qmax 7)
    int4 = {0.5: 0, 1.5: 2, 2.5: 2, 3.5: 4, 4.5: 4, 5.5: 6, 6.5: 6,
            -0.5: 0, -1.5: -2, -2.5: -2, -3.5: -4, -4.5: -4, -5.5: -6, -6.5: -6}
    for qmax, table in ((127, int8), (7, int4)):
        vals = list(table)
        x = np.zeros((1, 32 * ((len(vals) + 1 + 31) // 32)), np.float32)
        x[0, 0] = qmax                                     # the group's absmax: scale 1
        x[0, 1:1 + len(vals)] = vals
        codes, s = encode_groups_int(x, qmax)
        assert s[0, 0] == np.float16(1.0)
        assert codes[0, 0] == qmax
        assert [int(c) for c in codes[0, 1:1 + len(vals)]] == [table[v] for v in vals], qmax


@pytest.mark.parametrize("qmax", [127, 7])
def test_int_groups_equal_the_generator(qmax):
    x = np.random.default_rng(11).standard_normal((8, 64, 128)).astype(np.float16).astype(np.float32)
    c_gen, s_gen = senc.encode_int_g32(x, qmax)
    for i in range(8):
        c, s = encode_groups_int(x[i], qmax)
        assert np.array_equal(c, c_gen[i]) and np.array_equal(s, s_gen[i])


def test_affine2_closed_forms():
    """INT2 (unsigned affine, 2 bits): hand-worked groups."""
    x = np.zeros((3, 32), np.float32)
    # group 0: min -1.5, max 1.5 -> z = -1.5, s = 1; the grid points and the
    # three midpoints (quotients 0.5, 1.5, 2.5 go to the even code)
    x[0, :7] = [-1.5, -0.5, 0.5, 1.5, -1.0, 0.0, 1.0]
    x[0, 7:] = 0.5
    # group 1: all equal -> s = 1, every code 0, decodes to the value exactly
    x[1, :] = 2.5
    # group 2: min 0.25 is exact in fp16, max 6.25 -> s = 2
    x[2, :] = 0.25
    x[2, 3], x[2, 4] = 6.25, 3.25
    codes, s, z = encode_groups_affine2(x.reshape(1, 96))
    assert list(s[0]) == [1.0, 1.0, 2.0] and list(z[0]) == [-1.5, 2.5, 0.25]
    assert list(codes[0, :7]) == [0, 1, 2, 3, 0, 2, 2]
    assert np.all(codes[0, 32:64] == 0)
    assert codes[0, 64 + 3] == 3 and codes[0, 64 + 4] == 2 and codes[0, 64] == 0
    # round trip within half a step on random groups
    rng = np.random.default_rng(2)
    y = (rng.standard_normal((16, 128)) * rng.uniform(0.1, 5, (16, 1))).astype(np.float16).astype(np.float32)
    c, s, z = encode_groups_affine2(y)
    dec = z.astype(np.float64).repeat(32, 1) + c * s.astype(np.float64).repeat(32, 1)
    step = s.astype(np.float64).repeat(32, 1)
    assert np.all(np.abs(dec - y) <= 0.5 * step * (1 + 1e-3) + 1e-3 * np.abs(y))
    assert c.min() == 0 and c.max() == 3


def test_sign1_closed_forms():
    """BIT1: the sign bit (x < 0) and the exact mean magnitude."""
    x = np.zeros((1, 96), np.float32)
    x[0, :32] = np.where(np.arange(32) % 3 == 0, -0.75, 0.75)       # |x| = 0.75 -> s = 0.75
    x[0, 32:64] = 0.0                                                 # all zero -> s = 0
    x[0, 64:96] = np.arange(1, 33, dtype=np.float32) / 16            # mean (32*33/2)/16/32 = 1.03125
    bits, s = encode_groups_sign1(x)
    assert list(s[0]) == [0.75, 0.0, 1.03125]
    assert np.array_equal(bits[0, :32], (np.arange(32) % 3 == 0).astype(np.uint8))
    assert np.all(bits[0, 32:] == 0)
    neg0 = np.full((1, 32), -0.0, np.float32)                        # -0 is not below zero
    assert np.all(encode_groups_sign1(neg0)[0] == 0)


@pytest.mark.parametrize("src", [np.float16, "bf16"])
def test_affine2_and_sign1_equal_the_generator(src):
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((4, 32, 128)) * rng.uniform(0.01, 30, (4, 32, 1))).astype(np.float32)
    if src == "bf16":
        x = torch.from_numpy(x * 1e3).to(torch.bfloat16).to(torch.float32).numpy()
    else:
        x = x.astype(np.float16).astype(np.float32)
    gc, gs, gz = senc.encode_affine2_g32(x)
    bc, bs = senc.encode_sign1_g32(x)
    for i in range(4):
        c, s, z = encode_groups_affine2(x[i])
        assert np.array_equal(c, gc[i]) and np.array_equal(s, gs[i]) and np.array_equal(z, gz[i])
        b, s1 = encode_groups_sign1(x[i])
        assert np.array_equal(b, bc[i]) and np.array_equal(s1, bs[i])


def fp16_page(rng, hkv, P, D, codec=FP16):
    """Random fp16 values [2 planes][Hkv][P][D] and their 16-bit plane bytes."""
    x = (rng.standard_normal((2, 1, hkv, P, D)) * 2).astype(np.float16).astype(np.float32)
    k, _ = slay.encode_plane(x[0], codec, v_order=False)
    v, _ = slay.encode_plane(x[1], codec, v_order=True)
    return x[:, 0], k[0], v[0]


@pytest.mark.parametrize("dst", [FP8, INT8, INT4, BF16, INT2, BIT1])
@pytest.mark.parametrize("D", [64, 128])
def test_encode_page_equals_the_generator_bytes(dst, D):
    rng = np.random.default_rng(D + dst)
    hkv, P = 2, 32
    x, kb, vb = fp16_page(rng, hkv, P, D)
    pk = slay.plane_bytes(FP16, hkv, P, D)
    dk = slay.plane_bytes(dst, hkv, P, D)
    pool = np.zeros(2 * pk + 2 * dk, np.uint8)
    pool[:pk], pool[pk:2 * pk] = kb, vb
    out, scales = encode_page(pool, 0, pk, FP16 | FP16 << 4, 2 * pk, 2 * pk + dk, dst | dst << 4, hkv, P, D)
    assert np.array_equal(out[:2 * pk], pool[:2 * pk])                # source untouched
    gk, sk = slay.encode_plane(x[0][None], dst, v_order=False)
    gv, sv = slay.encode_plane(x[1][None], dst, v_order=True)
    assert np.array_equal(out[2 * pk: 2 * pk + dk], gk[0])
    assert np.array_equal(out[2 * pk + dk:], gv[0])
    if dst == FP8:
        assert np.array_equal(scales[:, 0], sk[0]) and np.array_equal(scales[:, 1], sv[0])
    else:
        assert np.all(scales == 1.0)
    # the read path's decoder sees values near the source
    for h in range(hkv):
        for i, (off, is_v) in enumerate(((2 * pk, False), (2 * pk + dk, True))):
            val = plane_values(out, off, dst, hkv, P, D, h, scales[h, i], is_v, P)
            if dst == BIT1:       # sign times the group's mean magnitude: the signs survive
                assert np.all((val < 0) == (x[i][h] < 0))
                continue
            tol = {FP8: 0.07, INT8: 0.01, INT4: 0.2, BF16: 0.01, INT2: 0.5}[dst]
            assert np.max(np.abs(val - x[i][h])) <= tol * np.max(np.abs(x[i][h]))


@pytest.mark.parametrize("codec", [FP16, BF16])
def test_append_token_changes_exactly_one_slot(codec):
    rng = np.random.default_rng(7 + codec)
    hkv, P, D = 2, 32, 64
    x, kb, vb = fp16_page(rng, hkv, P, D, codec)
    pk = slay.plane_bytes(codec, hkv, P, D)
    pool = np.concatenate([kb, vb])
    k_new = rng.standard_normal((hkv, D)).astype(np.float16)
    v_new = rng.standard_normal((hkv, D)).astype(np.float16)
    slot = 21
    out = append_token(pool, 0, pk, codec | codec << 4, hkv, P, D, slot, k_new, v_new)
    changed = np.flatnonzero(out != pool)
    assert changed.size <= 2 * 2 * hkv * D                            # two bytes per element at most
    for h in range(hkv):
        for off, is_v, new, old in ((0, False, k_new, x[0]), (pk, True, v_new, x[1])):
            val = plane_values(out, off, codec, hkv, P, D, h, 1.0, is_v, P)
            want = new[h].astype(np.float32)
            if codec == BF16:
                want = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
            assert np.array_equal(val[slot], want.astype(np.float64))
            keep = np.arange(P) != slot
            before = old[h][keep]
            if codec == BF16:
                before = torch.from_numpy(np.ascontiguousarray(before)).to(torch.bfloat16).float().numpy()
            assert np.array_equal(val[keep], before.astype(np.float64))
    with pytest.raises(ValueError):
        append_token(pool, 0, pk, FP8 | FP8 << 4, hkv, P, D, slot, k_new, v_new)


def test_append_then_whole_page_matches_the_generator():
    """Filling an empty FP16 page token by token gives the generator's page."""
    rng = np.random.default_rng(17)
    hkv, P, D = 2, 16, 64
    x, kb, vb = fp16_page(rng, hkv, P, D)
    pk = slay.plane_bytes(FP16, hkv, P, D)
    pool = np.zeros(2 * pk, np.uint8)
    for t in range(P):
        pool = append_token(pool, 0, pk, FP16 | FP16 << 4, hkv, P, D, t,
                            x[0][:, t, :].astype(np.float16), x[1][:, t, :].astype(np.float16))
    assert np.array_equal(pool[:pk], kb) and np.array_equal(pool[pk:], vb)
