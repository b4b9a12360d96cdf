"""Pins of the cache-append oracle (CPU only): the rotation, the E4M3 encoder
written from the format definition, the FP8 write recipe, and the append
seen through decode."""

import numpy as np
import pytest

from oracle import cache_append as A
from oracle import mla_oracle as O
from mla_latent_kv_absorb_amd import inputs as I


def test_rotation_hand_values_and_properties():
    # (1, 0) by 90 degrees -> (0, 1); (3, 4) by 180 degrees -> (-3, -4); angle 0 is the identity
    out = A.rope_rotate([1.0, 0.0, 3.0, 4.0, 5.0, -2.0], [0.0, -1.0, 1.0], [1.0, 0.0, 0.0])
    np.testing.assert_allclose(out, [0.0, 1.0, -3.0, -4.0, 5.0, -2.0], atol=1e-15)
    rng = np.random.default_rng(1)
    x = rng.standard_normal(64)
    th1, th2 = rng.uniform(-3, 3, 32), rng.uniform(-3, 3, 32)
    y = A.rope_rotate(x, np.cos(th1), np.sin(th1))
    # each pair keeps its length; two rotations add their angles
    np.testing.assert_allclose(np.hypot(y[0::2], y[1::2]), np.hypot(x[0::2], x[1::2]), rtol=1e-14)
    np.testing.assert_allclose(A.rope_rotate(y, np.cos(th2), np.sin(th2)),
                               A.rope_rotate(x, np.cos(th1 + th2), np.sin(th1 + th2)), atol=1e-13)


def test_rotated_dot_depends_on_offset_only():
    """With angles position * theta_i, a rotated query and a rotated key score
    the same for every pair of positions at the same distance: the property
    that makes the rotation a relative-position signal."""
    rng = np.random.default_rng(2)
    d = 64
    theta = 10000.0 ** (-np.arange(0, d, 2) / d)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    rot = lambda v, p: A.rope_rotate(v, np.cos(p * theta), np.sin(p * theta))
    base = rot(q, 7) @ rot(k, 3)
    for m, n in ((11, 7), (104, 100), (4, 0)):
        assert abs(rot(q, m) @ rot(k, n) - base) < 1e-10


def test_e4m3_encoder_from_format_definition():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.e4m3_to_f64(codes)
    # every value encodes back to its own code (except -0, which encodes as +0)
    back = A.encode_e4m3_nearest(vals)
    np.testing.assert_array_equal(back[codes != 0x80], codes[codes != 0x80])
    assert A.encode_e4m3_nearest([-0.0])[0] == 0
    # midpoints go to the even code: 1.0625 lies between 1.0 (0x38) and 1.125
    # (0x39); 1.1875 between 1.125 (0x39) and 1.25 (0x3A)
    np.testing.assert_array_equal(A.encode_e4m3_nearest([1.0625, 1.1875, -1.0625]), [0x38, 0x3A, 0xB8])
    # just off a midpoint goes to the nearer value; the top of the range is 448
    np.testing.assert_array_equal(A.encode_e4m3_nearest([1.0626, 448.0, 440.0]), [0x39, 0x7E, 0x7E])
    # the subnormal step is 2^-9: 0.75 * 2^-9 -> code 1, 0.25 * 2^-9 -> 0
    np.testing.assert_array_equal(A.encode_e4m3_nearest([0.75 * 2.0 ** -9, 0.25 * 2.0 ** -9]), [1, 0])
    with pytest.raises(ValueError):
        A.encode_e4m3_nearest([500.0])


def test_fp8_write_recipe():
    rng = np.random.default_rng(3)
    c = rng.standard_normal(512).astype(np.float32)
    codes, scales = A.quantize_token(c, 1)
    assert scales[0] == np.float32(np.max(np.abs(c))) / np.float32(448.0)
    vals = O.e4m3_to_f64(codes)
    assert np.max(np.abs(vals)) == 448.0                      # the largest magnitude maps to 448
    # each stored value is within half an E4M3 step of the quotient
    q = c / scales[0]
    assert np.all(np.abs(vals - q) <= np.maximum(np.abs(q) * 2.0 ** -4, 2.0 ** -10) + 1e-12)
    # group scales: one per 128 channels, each group reaching 448
    codes4, scales4 = A.quantize_token(c, 4)
    for g in range(4):
        part = c[128 * g:128 * (g + 1)]
        assert scales4[g] == np.float32(np.max(np.abs(part))) / np.float32(448.0)
        assert np.max(np.abs(O.e4m3_to_f64(codes4[128 * g:128 * (g + 1)]))) == 448.0
    # an all-zero latent stores zeros with scale 1
    z_codes, z_scales = A.quantize_token(np.zeros(512, np.float32), 4)
    assert np.all(z_codes == 0) and np.all(z_scales == 1.0)
    # the generator's per-token quantiser follows the same recipe
    g_codes, g_scales = I.quantize_fp8_per_token(c[None, :])
    np.testing.assert_array_equal(g_codes[0], codes)
    assert g_scales[0] == scales[0]


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], np.float32)
    np.testing.assert_array_equal(A.bf16_round(x), np.array([1.0, 1.0 + 2.0 ** -6, 1.0], np.float32))


def test_appended_token_is_what_decode_reads():
    """Appending token T with its rotation, then decoding over T + 1 positions,
    equals decoding over the logical arrays with that token added."""
    rng = np.random.default_rng(4)
    T, D_C, D_R, H = 9, 16, 8, 3
    c = rng.standard_normal((T, D_C)).astype(np.float32)
    kr = rng.standard_normal((T, D_R)).astype(np.float32)
    c_new, k_new = rng.standard_normal(D_C).astype(np.float32), rng.standard_normal(D_R).astype(np.float32)
    th = T * 10000.0 ** (-np.arange(0, D_R, 2) / D_R)
    pay, krot, _ = A.append_token(c_new, k_new, np.cos(th), np.sin(th), "f32")
    ql, qr = rng.standard_normal((H, D_C)), rng.standard_normal((H, D_R))
    got = O.latent_decode(ql, qr, np.vstack([c, pay]), np.vstack([kr, krot]), 0.3)
    want = O.latent_decode(ql, qr, np.vstack([c, c_new]), np.vstack([kr, A.rope_rotate(k_new, np.cos(th), np.sin(th))]), 0.3)
    np.testing.assert_allclose(got[0], want[0], rtol=1e-6, atol=1e-6)
    # without the rotation the result differs: the rotation is not dropped
    bad = O.latent_decode(ql, qr, np.vstack([c, c_new]), np.vstack([kr, k_new]), 0.3)
    assert not np.allclose(got[1], bad[1], rtol=1e-6, atol=1e-6)
