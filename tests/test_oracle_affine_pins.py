"""Pins of the group-affine oracle (rotated keys, group-64 affine codes with
fp16 scale and bias; mlx-turboquant README, "Quantize the KV cache", "How it
plugs in", "Memory footprint over long context").

Each pin checks the oracle against something other than its own formula:
a brute-force nearest-level search, hand-worked groups, the error bound of
a uniform grid, attention formed densely in the original frame, and the
README's byte table."""

import json
import math
import os

import numpy as np
import pytest

import oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f16(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def _ulp16(x):
    x = np.abs(np.asarray(x, np.float64)).astype(np.float16)
    return (np.nextafter(x, np.float16(np.inf)) - x).astype(np.float64)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_affine_code_is_nearest_level_of_stored_grid(bits):
    rng = np.random.default_rng(10 + bits)
    y = rng.standard_normal((200, 128)) * rng.uniform(0.1, 3.0, (200, 1))
    codes, s, b = o.affine_quantize_group_rows(y, bits)
    L = (1 << bits) - 1
    levels = b[..., None] + s[..., None] * np.arange(L + 1)          # [200][2][L+1]
    yg = y.reshape(200, 2, 64)
    dist = np.abs(yg[..., None] - levels[:, :, None, :])              # [200][2][64][L+1]
    best = dist.argmin(axis=-1)
    srt = np.sort(dist, axis=-1)
    clear = (srt[..., 1] - srt[..., 0]) > 1e-9
    assert np.array_equal(codes.reshape(200, 2, 64)[clear], best[clear])
    # the grid spans the group up to the fp16 rounding of its two numbers
    assert np.all(np.abs(b - yg.min(-1)) <= _ulp16(yg.min(-1)) / 2 + 1e-300)
    top = b + L * s
    tol = L * _ulp16((yg.max(-1) - yg.min(-1)) / L) / 2 + _ulp16(yg.min(-1)) / 2
    assert np.all(np.abs(top - yg.max(-1)) <= tol * 1.0001)


def test_affine_hand_worked_groups():
    # 2 bits, values 0..3 repeated: min 0, max 3 -> scale 1, bias 0, codes = values
    y = np.tile(np.array([0.0, 1.0, 2.0, 3.0]), 32)[None, :]
    codes, s, b = o.affine_quantize_group_rows(y, 2)
    assert np.array_equal(codes[0], y[0].astype(np.uint8))
    assert s.tolist() == [[1.0, 1.0]] and b.tolist() == [[0.0, 0.0]]
    # 4 bits on [-1, 2]: scale 3/15 = 0.2 (fp16 0.199951171875), bias -1;
    # 0.5 sits at 1.5 / 0.19995 = 7.5018 -> code 8; 2.0 clamps to 15
    y = np.full((1, 64), 0.5)
    y[0, 0], y[0, 1] = -1.0, 2.0
    codes, s, b = o.affine_quantize_group_rows(y, 4, group=64)
    assert s[0, 0] == 0.199951171875 and b[0, 0] == -1.0
    assert codes[0, 0] == 0 and codes[0, 1] == 15 and codes[0, 2] == 8
    # a constant group: scale 0, every code 0, dequantized to fp16(c)
    y = np.full((1, 128), 0.1)
    codes, s, b = o.affine_quantize_group_rows(y, 4)
    assert np.all(codes == 0) and np.all(s == 0)
    assert np.all(o.affine_dequant(codes, s, b) == _f16(0.1))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_affine_error_within_half_step(bits):
    rng = np.random.default_rng(3)
    y = rng.standard_normal((500, 256))
    codes, s, b = o.affine_quantize_group_rows(y, bits)
    yh = o.affine_dequant(codes, s, b)
    step = np.repeat(s, 64, axis=-1)
    L = (1 << bits) - 1
    # inside the stored grid the error is at most half a step; at the ends
    # the fp16 rounding of the bias and of L * scale adds at most an ulp each
    slack = np.repeat(_ulp16(b) + L * _ulp16(s), 64, axis=-1)
    assert np.all(np.abs(y - yh) <= step / 2 + slack + 1e-15)


@pytest.mark.parametrize("G", [1, 3])
def test_affine_attention_equals_dense_softmax_in_original_frame(G):
    rng = np.random.default_rng(7)
    d, n, Hkv, seed = 128, 37, 2, 99
    k = rng.standard_normal((1, Hkv, n, d))
    v = rng.standard_normal((1, Hkv, n, d))
    q = rng.standard_normal((1, Hkv * G, d))
    c = o.affine_encode_kv(k, v, bits_k=4, bits_v=4, seed=seed)
    got = o.affine_attend(q, c, n, d=d, seed=seed, bits_k=4, bits_v=4, Hkv=Hkv)
    R = o.rotation_matrix(seed, d)                      # dense Sylvester form
    for g in range(Hkv):
        ky = np.zeros((n, d))
        vh = np.zeros((n, d))
        for j in range(n):                              # element by element
            kc = o.unpack_codes(c["kc"][0, g, j], 4, d)
            vc = o.unpack_codes(c["vc"][0, g, j], 4, d)
            for i in range(d):
                grp = i // 64
                ky[j, i] = float(c["ks"][0, g, j, grp]) * kc[i] + float(c["kb"][0, g, j, grp])
                vh[j, i] = float(c["vs"][0, g, j, grp]) * vc[i] + float(c["vb"][0, g, j, grp])
        k_hat = ky @ R                                  # R^T y_hat, row form
        for h in range(g * G, (g + 1) * G):
            s = k_hat @ q[0, h] / math.sqrt(d)
            p = np.exp(s - s.max())
            want = (p / p.sum()) @ vh
            assert np.allclose(got[0, h], want, rtol=0, atol=1e-12)
        # and the dequantized keys stay close to the true keys (4-bit grid over
        # about 6 standard deviations: rms error about 0.4 / sqrt(12))
        rel = np.linalg.norm(k_hat - k[0, g], axis=-1) / np.linalg.norm(k[0, g], axis=-1)
        assert rel.max() < 0.2


def test_affine_record_matches_readme_byte_table():
    with open(os.path.join(GOLD, "kv_bytes_per_token.json")) as f:
        g = json.load(f)["kb_per_token"]
    E = int(g["fp16"] * 1024 / 2 / 2)             # K (or V) elements per token
    vectors = E // 128                               # 128-long K (or V) vectors per token
    assert round(vectors * o.affine_cache_bytes_per_token(128, 4, 4) / 1024, 1) == g["affine4_g64"]
    assert round(vectors * o.affine_cache_bytes_per_token(128, 8, 8) / 1024, 1) == g["affine8_g64"]


def test_affine_band_flags_half_integers_only():
    y = np.zeros((2, 64))
    y[:, 1] = 3.0                                     # 2 bits: scale 1, bias 0
    y[0, 2] = 1.5                                     # exactly between two levels
    y[1, 2] = 1.25
    bad = o.affine_code_ambiguous(y, 2)
    assert bad.tolist() == [True, False]
