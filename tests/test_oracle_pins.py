"""Pins for the CPU oracle: each test ties an oracle function to something
other than itself (closed forms, library routines, brute force on tiny
inputs, published generator values, statistics, values printed on the pages).
CPU only."""

import json
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg

import oracle as o
import seeded_inputs as si

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------- generator

def test_splitmix64_published_values():
    # Reference outputs of SplitMix64 from state 0 (Vigna's splitmix64.c).
    assert o.splitmix64(0, 4) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                  0x06C45D188009454F, 0xF88BB8A8724C81EC]


def test_signs_follow_top_bit_and_are_balanced():
    s = o.signs(0, 4)
    assert list(s) == [-1.0, 1.0, 1.0, -1.0]   # top bits of the outputs above
    big = o.signs(12345, 4096)
    assert set(np.unique(big)) == {-1.0, 1.0}
    assert abs(big.mean()) < 0.06
    assert not np.array_equal(o.signs(0, 256), o.signs(1, 256))


# ---------------------------------------------------------------- rotation

@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_equals_library_hadamard(d):
    """P2: the butterfly FWHT is H_d x for SciPy's Sylvester Hadamard."""
    rng = np.random.default_rng(d)
    x = rng.standard_normal((3, d))
    H = scipy.linalg.hadamard(d).astype(np.float64)
    np.testing.assert_allclose(o.fwht(x), x @ H.T, rtol=0, atol=1e-12)
    assert np.array_equal(o.hadamard_sylvester(d), H)
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H, d * np.eye(d))


@pytest.mark.parametrize("d", [8, 128, 256])
@pytest.mark.parametrize("seed", [0, 7])
def test_rht_is_orthogonal_and_matches_dense(d, seed):
    """P1: R^T R = I, R^T (R x) = x, inner products preserved."""
    eye = np.eye(d)
    R = o.rht(eye, seed).T                     # column j = R e_j
    Rdense = scipy.linalg.hadamard(d) * o.signs(seed, d)[None, :] / math.sqrt(d)
    np.testing.assert_allclose(R, Rdense, atol=1e-15)
    assert np.abs(R.T @ R - eye).max() <= 1e-14
    rng = np.random.default_rng(seed + d)
    x, y = rng.standard_normal((2, 5, d))
    np.testing.assert_allclose(o.rht_inverse(o.rht(x, seed), seed), x, atol=1e-13)
    lhs = (o.rht(x, seed) * o.rht(y, seed)).sum(-1)
    np.testing.assert_allclose(lhs, (x * y).sum(-1), atol=1e-12)


# ---------------------------------------------------------------- codebook

@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_lloyd_max_conditions_by_quadrature(bits):
    """P3: centroid condition (by numerical integration, not the closed form
    the iteration uses), midpoint condition, symmetry, middle threshold 0."""
    c, t = o.lloyd_max(bits)
    assert len(c) == 2 ** bits and len(t) == 2 ** bits - 1
    assert np.all(np.diff(c) > 0)
    edges = [-np.inf] + list(t) + [np.inf]
    pdf = lambda z: math.exp(-z * z / 2) / math.sqrt(2 * math.pi)
    for k in range(len(c)):
        a, b = edges[k], edges[k + 1]
        m0 = scipy.integrate.quad(pdf, a, b, epsabs=1e-15, epsrel=1e-13)[0]
        m1 = scipy.integrate.quad(lambda z: z * pdf(z), a, b, epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(m1 / m0 - c[k]) < 1e-10
    np.testing.assert_allclose(t, (c[1:] + c[:-1]) / 2, rtol=0, atol=1e-15)
    assert np.array_equal(c, -c[::-1])
    assert t[len(t) // 2] == 0.0


def test_codebook_closed_form_one_bit():
    """P4: b=1 is +-sqrt(2/pi) with MSE 1 - 2/pi."""
    c, t = o.lloyd_max(1)
    np.testing.assert_allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-14)
    assert abs(o.codebook_mse(1) - (1 - 2 / math.pi)) < 1e-13


@pytest.mark.parametrize("bits,cpos,tpos,mse", [
    # Gaussian Lloyd-Max (Max, "Quantizing for minimum distortion", 1960),
    # positive half; the classic table is accurate to about 3 decimals.
    (2, [0.4528, 1.510], [0.9816], 0.1175),
    (3, [0.2451, 0.7560, 1.344, 2.152], [0.5006, 1.050, 1.748], 0.03455),
    (4, [0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733],
     [0.2582, 0.5224, 0.7996, 1.099, 1.437, 1.844, 2.401], 0.009497),
])
def test_codebook_matches_classic_table(bits, cpos, tpos, mse):
    c, t = o.lloyd_max(bits)
    half = len(c) // 2
    np.testing.assert_allclose(c[half:], cpos, atol=1.5e-3)
    np.testing.assert_allclose(t[half:], tpos, atol=1.5e-3)
    assert abs(o.codebook_mse(bits) - mse) / mse < 2e-3


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_mse_by_quadrature(bits):
    c, t = o.lloyd_max(bits)
    edges = [-np.inf] + list(t) + [np.inf]
    pdf = lambda z: math.exp(-z * z / 2) / math.sqrt(2 * math.pi)
    total = sum(scipy.integrate.quad(lambda z: (z - c[k]) ** 2 * pdf(z), edges[k],
                                     edges[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
                for k in range(len(c)))
    assert abs(total - o.codebook_mse(bits)) < 1e-12


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_is_nearest_centroid(bits):
    """P5: the threshold count equals brute-force nearest centroid off ties;
    a value exactly on a threshold takes the upper code."""
    c, t = o.lloyd_max(bits)
    rng = np.random.default_rng(bits)
    z = rng.standard_normal(20000) * 1.5
    codes = o.quantize(z, t)
    brute = np.array([min(range(len(c)), key=lambda k: abs(zz - c[k])) for zz in z])
    assert np.array_equal(codes, brute)
    assert list(o.quantize(t, t)) == list(range(1, len(c)))
    assert o.quantize(np.array([0.0]), t)[0] == 2 ** (bits - 1)


# ------------------------------------------------------ decision bands
# The parity tests accept either adjacent code for a coordinate whose
# scaled rotated value z lies within 1e-6 of a threshold (z units), and
# either sign bit for a QJL coordinate with |w| < 1e-6 ||r||. These pins tie
# the two band helpers to that definition: fixed points just inside and
# outside the band, and the band equals the set where moving z (or w) by
# the band half-width changes the pinned quantizer's code (or the sign).

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_boundary_mask_is_the_1e6_band_in_z_units(bits):
    c, t = o.lloyd_max(bits)
    inside = np.concatenate([t - 5e-7, t + 5e-7])
    outside = np.concatenate([t - 2e-6, t + 2e-6])
    assert o.boundary_mask(inside, t).all()
    assert not o.boundary_mask(outside, t).any()
    assert not o.boundary_mask(c, t).any()               # cell centres
    assert o.boundary_mask(np.array([0.0, -3e-7, 9e-7]), t).all()   # t_mid = 0
    rng = np.random.default_rng(40 + bits)
    z = np.concatenate([t[rng.integers(0, len(t), 20000)] + rng.uniform(-4e-6, 4e-6, 20000),
                        rng.standard_normal(20000) * 1.5])
    eps = 1e-6
    moved = o.quantize(z + eps, t) != o.quantize(z - eps, t)
    assert np.array_equal(o.boundary_mask(z, t), moved)
    assert 0.1 < moved.mean() < 0.9
    # a [rows][d] array is flagged per coordinate
    zz = z[:1280].reshape(10, 128)
    assert np.array_equal(o.boundary_mask(zz, t), moved[:1280].reshape(10, 128))


def test_qjl_boundary_mask_is_the_band_relative_to_the_residual_norm():
    rn = np.array([1e-3, 1.0, 50.0])                     # ||r|| per row
    inside = np.array([[0.5e-6, -0.5e-6, 0.0, 0.9e-6]]) * rn[:, None]
    outside = np.array([[2e-6, -2e-6, 1.1e-6, -5.0]]) * rn[:, None]
    assert o.qjl_boundary_mask(inside, rn).all()
    assert not o.qjl_boundary_mask(outside, rn).any()
    rng = np.random.default_rng(44)
    w = rng.uniform(-4e-6, 4e-6, (3, 4096)) * rn[:, None]
    band = 1e-6 * rn[:, None]
    flips = (w + band < 0) != (w - band < 0)
    assert np.array_equal(o.qjl_boundary_mask(w, rn), flips)
    assert 0.1 < flips.mean() < 0.9


# ------------------------------------------------------------------ encode

@pytest.mark.parametrize("bits,d", [(2, 256), (3, 128), (4, 128)])
def test_encode_distortion_matches_codebook_mse(bits, d):
    """P6: on iid Gaussian rows the rotated, normalized coordinates quantize
    with the Lloyd-Max distortion (within 3%)."""
    rng = np.random.default_rng(100 + bits)
    x = rng.standard_normal((3000, d))
    enc = o.encode_vectors(x, 0, bits, "f32")
    c, _ = o.lloyd_max(bits)
    mse = ((enc["z"] - c[enc["codes"]]) ** 2).mean()
    assert abs(mse / o.codebook_mse(bits) - 1) < 0.03
    np.testing.assert_allclose((enc["z"] ** 2).sum(-1), d, rtol=1e-12)


def test_encode_zero_vector_and_norm_rounding():
    x = np.zeros((1, 128))
    enc = o.encode_vectors(x, 0, 3, "f16")
    assert np.all(enc["codes"] == 4) and enc["norm"][0] == 0.0
    # norm rounding: nearest-even in fp16
    v = np.zeros((1, 128)); v[0, 0] = 1.0 + 2 ** -11   # midpoint 1 .. 1+2^-10
    assert o.encode_vectors(v, 0, 3, "f16")["norm"][0] == 1.0
    v[0, 0] = 1.0 + 3 * 2 ** -11                         # midpoint, rounds to even
    assert o.encode_vectors(v, 0, 3, "f16")["norm"][0] == 1.0 + 2 * 2 ** -10
    assert o.norm_ambiguous(np.array([1.0 + 2 ** -11]), "f16")[0]
    assert not o.norm_ambiguous(np.array([1.0 + 2 ** -12]), "f16")[0]


def test_encode_equals_dense_rotation_brute_force():
    d, bits = 16, 3
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, d))
    R = o.rotation_matrix(3, d)
    enc = o.encode_vectors(x, 3, bits, "f32")
    c, t = o.lloyd_max(bits)
    for row, codes in zip(x, enc["codes"]):
        n = math.sqrt(sum(v * v for v in row))
        z = math.sqrt(d) * (R @ row) / n
        want = [sum(1 for tk in t if zi >= tk) for zi in z]
        assert list(codes) == want


# ----------------------------------------------------------------- packing

def test_pack_hand_worked_examples():
    g = _gold("pack_example.json")
    assert list(o.pack_codes(np.array(g["codes"]), 3)) == g["bytes"]
    assert list(o.pack_codes(np.array(g["bits2"]["codes"]), 2)) == g["bits2"]["bytes"]
    assert list(o.pack_codes(np.array(g["bits4"]["codes"]), 4)) == g["bits4"]["bytes"]


@pytest.mark.parametrize("bits,d", [(2, 128), (3, 128), (4, 128), (2, 256), (3, 256), (4, 256)])
def test_pack_matches_bit_loop_and_roundtrips(bits, d):
    rng = np.random.default_rng(bits * d)
    codes = rng.integers(0, 2 ** bits, size=(7, d)).astype(np.uint8)
    packed = o.pack_codes(codes, bits)
    assert packed.shape == (7, d * bits // 8)
    assert (d * bits // 8) % 16 == 0            # records are 16-byte multiples
    for r in range(7):
        acc = 0
        for i in range(d):
            acc |= int(codes[r, i]) << (bits * i)
        assert bytes(packed[r]) == acc.to_bytes(d * bits // 8, "little")
    assert np.array_equal(o.unpack_codes(packed, bits, d), codes)


def test_sign_words_layout():
    bits01 = np.zeros(128, np.uint8)
    bits01[[0, 31, 32, 127]] = 1
    words = o.pack_signs(bits01).view("<u4")
    assert list(words) == [1 | (1 << 31), 1, 0, 1 << 31]
    assert np.array_equal(o.unpack_signs(o.pack_signs(bits01), 128), bits01)


# ------------------------------------------------------------ QJL identity

def test_mse_bias_identity():
    """P8: <Rq, k_hat_rot> - <q, k> = -<Rq, r> exactly (README, QJL section)."""
    rng = np.random.default_rng(8)
    d = 128
    k = rng.standard_normal((50, d))
    q = 0.8 * k + 0.6 * rng.standard_normal((50, d))
    enc = o.encode_vectors(k, 0, 3, "f16")
    khat = o.dequant_rot(enc["codes"], enc["norm"], 3)
    rq = o.rht(q, 0)
    r = o.qjl_from_encoding(enc, 3, 1)["r"]
    lhs = (rq * khat).sum(-1) - (q * k).sum(-1)
    np.testing.assert_allclose(lhs, -(rq * r).sum(-1), atol=1e-12, rtol=0)


def test_qjl_constant_gaussian_projection_unbiased():
    """P9(i): with a Gaussian projection S (N(0,1) entries, m = d rows) in
    place of sqrt(d) R_2, the estimator with factor sqrt(QJL_CONST / d) is
    exactly unbiased for <Rq, r>: mean error within 4 standard errors."""
    rng = np.random.default_rng(9)
    d = 128
    k = rng.standard_normal(d)
    q = 0.8 * k + 0.6 * rng.standard_normal(d)
    enc = o.encode_vectors(k[None], 0, 3, "f16")
    r = o.qjl_from_encoding(enc, 3, 1)["r"][0]
    rq = o.rht(q[None], 0)[0]
    truth = rq @ r
    S = rng.standard_normal((4000, d, d))
    proj_q = (S @ rq) / math.sqrt(d)             # plays the role of R_2 R q
    sgn = np.where(S @ r < 0, -1.0, 1.0)
    est = math.sqrt(o.QJL_CONST / d) * np.linalg.norm(r) * (proj_q * sgn).sum(-1)
    err = est - truth
    se = err.std(ddof=1) / math.sqrt(len(err))
    assert abs(err.mean()) < 4 * se
    # the garbled reading sqrt(pi*d/2) would be off by a factor of d
    assert abs(truth) > 10 * se


@pytest.mark.slow
def test_qjl_rht_estimator_removes_bias():
    """P9(ii): the RHT_2 estimator the pages prescribe, on correlated pairs
    (q = 0.8 k + 0.6 eps, d=128, 3-bit keys) over many QJL seeds: the mean
    corrected bias is at most 0.1x the mean |MSE-only bias| (README, QJL
    section: the bias is removed to about zero)."""
    d, bits, pairs, seeds = 128, 3, 20, 2000
    rng = np.random.default_rng(10)
    k = rng.standard_normal((pairs, d))
    q = 0.8 * k + 0.6 * rng.standard_normal((pairs, d))
    enc = o.encode_vectors(k, 0, bits, "f16")
    khat = o.dequant_rot(enc["codes"], enc["norm"], bits)
    rq = o.rht(q, 0)
    truth = (q * k).sum(-1)
    mse_bias = (rq * khat).sum(-1) - truth
    r = enc["y"] - khat
    rn = o.round_norm(np.linalg.norm(r, axis=-1), "f16")
    corr_bias = np.zeros(pairs)
    for s in range(1, seeds + 1):
        w = o.rht(r, s)
        sgn = np.where(w < 0, -1.0, 1.0)
        est = math.sqrt(o.QJL_CONST / d) * rn * (o.rht(rq, s) * sgn).sum(-1)
        corr_bias += (mse_bias + est) / seeds
    assert np.abs(corr_bias).mean() <= 0.1 * np.abs(mse_bias).mean()


def test_qjl_sketch_zero_residual_and_polarity():
    out = o.qjl_sketch(np.zeros((1, 128)), 1)
    assert out["rnorm"][0] == 0 and not out["bits"].any()
    r = np.zeros((1, 128)); r[0, 5] = -2.0
    w = o.rht(r, 1)[0]
    assert np.array_equal(o.qjl_sketch(r, 1)["bits"][0], (w < 0).astype(np.uint8))


# --------------------------------------------------------------- attention

def _brute_attention(q, k, v, seed, bits_k, bits_v, norm_dtype, Hkv, tau,
                     qjl=False, qjl_seed=None):
    """Explicit matrices and loops: dequantize every token, two-pass softmax."""
    B, Hq, d = q.shape
    G = Hq // Hkv
    R = o.rotation_matrix(seed, d)
    ck, tk = o.lloyd_max(bits_k)
    cv, tv = o.lloyd_max(bits_v)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            khat, vhat, corr = [], [], []
            for j in range(k.shape[2]):
                kv = []
                for x, c, t in ((k[b, g, j], ck, tk), (v[b, g, j], cv, tv)):
                    n = math.sqrt(sum(e * e for e in x))
                    nr = float(np.float64(n).astype(o.turboquant._NORM_TYPES[norm_dtype]))
                    z = math.sqrt(d) * (R @ x) / n if n > 0 else np.zeros(d)
                    code = [sum(1 for tt in t if zi >= tt) for zi in z]
                    rot = np.array([nr * c[cc] / math.sqrt(d) for cc in code])
                    kv.append((rot, R @ x))
                khat.append(R.T @ kv[0][0])
                vhat.append(R.T @ kv[1][0])
                if qjl:
                    R2 = o.rotation_matrix(qjl_seed, d)
                    r = kv[0][1] - kv[0][0]
                    sig = np.where(R2 @ r < 0, -1.0, 1.0)
                    rn = float(np.float16(np.linalg.norm(r)))
                    corr.append(math.sqrt(math.pi / (2 * d)) * rn * ((R2 @ (R @ q[b, h])) @ sig))
            logits = [tau * (q[b, h] @ kh) + (tau * corr[j] if qjl else 0.0)
                      for j, kh in enumerate(khat)]
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            s = sum(w)
            out[b, h] = sum(wj / s * vh for wj, vh in zip(w, vhat))
    return out


@pytest.mark.parametrize("qjl", [False, True])
@pytest.mark.parametrize("N", [1, 5, 33])
def test_attention_matches_brute_force(N, qjl):
    """P7: dense and rotated-blocked modes against explicit brute force."""
    d, B, Hq, Hkv = 16, 2, 4, 2
    rng = np.random.default_rng(N)
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    kw = dict(seed=3, bits_k=3, bits_v=4, norm_dtype="f16")
    cache = o.encode_kv(k, v, qjl=qjl, qjl_seed=11, **kw)
    tau = 1 / math.sqrt(d)
    want = _brute_attention(q, k, v, 3, 3, 4, "f16", Hkv, tau, qjl, 11)
    dense = o.attend_dense(q, cache, d=d, seed=3, bits_k=3, bits_v=4, Hkv=Hkv,
                           qjl=qjl, qjl_seed=11)
    blocked = o.attend(q, cache, N, d=d, seed=3, bits_k=3, bits_v=4, Hkv=Hkv,
                       qjl=qjl, qjl_seed=11, block=4)
    np.testing.assert_allclose(dense, want, atol=1e-12, rtol=0)
    np.testing.assert_allclose(blocked, want, atol=1e-12, rtol=0)


def test_attention_special_cases():
    d = 32
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, d)) * 3
    k = rng.standard_normal((1, 1, 1, d))
    v = rng.standard_normal((1, 1, 1, d))
    cache = o.encode_kv(k, v, seed=0, bits_k=2, bits_v=2, norm_dtype="f16")
    vhat = o.rht_inverse(o.dequant_rot(o.unpack_codes(cache["vc"][0, 0], 2, d),
                                       cache["vn"][0, 0], 2), 0)
    out = o.attend(q, cache, 1, d=d, seed=0, bits_k=2, bits_v=2, Hkv=1)
    np.testing.assert_allclose(out[0, 0], vhat[0], atol=1e-14)   # N = 1
    # identical keys: uniform weights, output = mean of v_hat
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), 9, axis=2)
    v = rng.standard_normal((1, 1, 9, d))
    cache = o.encode_kv(k, v, seed=0, bits_k=3, bits_v=4, norm_dtype="f16")
    vhat = o.rht_inverse(o.dequant_rot(o.unpack_codes(cache["vc"][0, 0], 4, d),
                                       cache["vn"][0, 0], 4), 0)
    out = o.attend(q, cache, 9, d=d, seed=0, bits_k=3, bits_v=4, Hkv=1, block=2)
    np.testing.assert_allclose(out[0, 1], vhat.mean(0), atol=1e-13)


def test_attention_scale_and_merge():
    """Explicit scale; the LSE merge is exact for any block split."""
    d, N = 16, 40
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    cache = o.encode_kv(k, v, seed=1, bits_k=4, bits_v=3, norm_dtype="f32")
    a = o.attend(q, cache, N, d=d, seed=1, bits_k=4, bits_v=3, Hkv=1, scale=0.37, block=N)
    for blk in (1, 3, 13):
        b = o.attend(q, cache, N, d=d, seed=1, bits_k=4, bits_v=3, Hkv=1, scale=0.37, block=blk)
        np.testing.assert_allclose(a, b, atol=1e-13)
    dense = o.attend_dense(q, cache, d=d, seed=1, bits_k=4, bits_v=3, Hkv=1, scale=0.37)
    np.testing.assert_allclose(a, dense, atol=1e-13)


@pytest.mark.parametrize("qjl", [False, True])
def test_prefill_rows_equal_brute_force_over_their_prefix(qjl):
    """Causal prefill: query i of the chunk sits at position n_ctx - n_q + i
    and equals brute-force attention over tokens 0..that position."""
    d, B, Hq, Hkv, N, n_q = 16, 1, 4, 2, 21, 7
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, Hq, n_q, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    cache = o.encode_kv(k, v, seed=3, bits_k=3, bits_v=4, norm_dtype="f16", qjl=qjl,
                        qjl_seed=11)
    got = o.attend_prefill(q, cache, N, d=d, seed=3, bits_k=3, bits_v=4, Hkv=Hkv, qjl=qjl,
                           qjl_seed=11)
    tau = 1 / math.sqrt(d)
    for i in range(n_q):
        p = N - n_q + i
        want = _brute_attention(q[:, :, i], k[:, :, :p + 1], v[:, :, :p + 1], 3, 3, 4, "f16",
                                Hkv, tau, qjl, 11)
        np.testing.assert_allclose(got[:, :, i], want, atol=1e-12, rtol=0)


def test_prefill_special_cases():
    """The chunk's first query of a fresh cache sees token 0 only (output =
    v_hat_0); a one-query chunk is the decode step."""
    d, N = 32, 12
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 2, N, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    cache = o.encode_kv(k, v, seed=0, bits_k=2, bits_v=3, norm_dtype="f32")
    vhat = o.rht_inverse(o.dequant_rot(o.unpack_codes(cache["vc"][0, 0], 3, d),
                                       cache["vn"][0, 0], 3), 0)
    out = o.attend_prefill(q, cache, N, d=d, seed=0, bits_k=2, bits_v=3, Hkv=1)
    np.testing.assert_allclose(out[0, :, 0], np.repeat(vhat[:1], 2, axis=0), atol=1e-14)
    one = o.attend_prefill(q[:, :, 5:6], cache, N, d=d, seed=0, bits_k=2, bits_v=3, Hkv=1,
                           scale=0.3)
    dec = o.attend(q[:, :, 5], cache, N, d=d, seed=0, bits_k=2, bits_v=3, Hkv=1, scale=0.3)
    np.testing.assert_allclose(one[:, :, 0], dec, atol=1e-13)


@pytest.mark.parametrize("d", [16, 128, 256])
def test_sphere_density_has_unit_variance(d):
    """z = sqrt(d) u for u a coordinate of a uniform unit vector: E[z^2] =
    d E[u^2] = 1 exactly, which fixes the exponent (d-3)/2 of the density."""
    r = math.sqrt(d)
    z0 = scipy.integrate.quad(lambda z: o.sphere_density(z, d), -r, r, epsabs=1e-14)[0]
    z2 = scipy.integrate.quad(lambda z: z * z * o.sphere_density(z, d), -r, r, epsabs=1e-14)[0]
    assert abs(z2 / z0 - 1.0) < 1e-10


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 256])
def test_sphere_codebook_lloyd_max_conditions(bits, d):
    """Centroid condition by quadrature of the density itself (not the
    closed-form first moment the iteration uses), midpoint condition,
    antisymmetry, zero middle threshold."""
    c, t = o.lloyd_max(bits, d)
    L = 1 << bits
    assert len(c) == L and len(t) == L - 1
    np.testing.assert_allclose(c, -c[::-1], atol=0)
    assert t[L // 2 - 1] == 0.0
    np.testing.assert_allclose(t, (c[:-1] + c[1:]) / 2, atol=1e-15)
    edges = [-math.sqrt(d)] + list(t) + [math.sqrt(d)]
    for k in range(L):
        a, b = edges[k], edges[k + 1]
        m0 = scipy.integrate.quad(lambda z: o.sphere_density(z, d), a, b, epsabs=1e-14)[0]
        m1 = scipy.integrate.quad(lambda z: z * o.sphere_density(z, d), a, b, epsabs=1e-14)[0]
        assert abs(m1 / m0 - c[k]) < 1e-9


def test_sphere_codebook_limits_and_optimality():
    """Large d gives the N(0,1) codebook; on samples of the exact marginal
    (first coordinate of a uniform unit vector, drawn as g0 / sqrt(g0^2 +
    chi2_{d-1})) the finite-d codebook has the lower distortion."""
    # the finite-d correction shrinks like 1/d (4-bit: 0.044 at d 128)
    for bits in (2, 3, 4):
        np.testing.assert_allclose(o.lloyd_max(bits, 4096)[0], o.lloyd_max(bits)[0],
                                   atol=2e-3)
    d, n = 128, 4_000_000
    rng = np.random.default_rng(0)
    g0 = rng.standard_normal(n)
    z = math.sqrt(d) * g0 / np.sqrt(g0 * g0 + rng.chisquare(d - 1, n))
    cs, ts = o.lloyd_max(4, d)
    cg, tg = o.lloyd_max(4)
    diff = (z - cg[o.quantize(z, tg)]) ** 2 - (z - cs[o.quantize(z, ts)]) ** 2
    assert diff.mean() > 3 * diff.std() / math.sqrt(n)


def test_rotation_flattens_outliers():
    """P10 (outlier workload): rotation cuts max|z| and the 2-bit z-distortion."""
    w = si.WORKLOADS[3]
    _, k = si.kv_rows(w, si.T_K, 0, 0, 0, 4096)
    k = k.astype(np.float64)
    c, t = o.lloyd_max(2)
    n = np.linalg.norm(k, axis=-1, keepdims=True)
    z_raw = math.sqrt(w.d) * k / n
    z_rot = o.encode_vectors(k, 0, 2, "f16")["z"]
    mse = lambda z: ((z - c[o.quantize(z, t)]) ** 2).mean()
    assert np.abs(z_raw).max() / np.abs(z_rot).max() >= 2.5
    assert mse(z_raw) / mse(z_rot) >= 4.0


# ------------------------------------------------------- rules and bytes

def test_enable_rule_and_split_truth_table():
    g = _gold("enable_rule.json")
    for bits, scheme, want in g["enabled"]:
        assert o.turboquant_enabled(bits, scheme) is want, (bits, scheme)
    for bits, scheme, bk, bv in g["split_pinned_by_pages"]:
        assert o.bits_split(bits, scheme) == (bk, bv)
    assert o.bits_split(4, "turboquant") == (4, 4)
    assert o.bits_split(4.0) is None
    assert o.bits_split(2.5) == (2, 3)


def test_byte_accounting_reproduces_readme_table():
    """P12: format arithmetic reproduces the README's KB/token column."""
    g = _gold("kv_bytes_per_token.json")["kb_per_token"]
    E = int(g["fp16"] * 1024 / 2 / 2)              # K (or V) elements per token
    assert E == 28672
    kb = lambda x: round(x / 1024, 1)
    assert kb(o.fp16_bytes_per_token(2 * E)) == g["fp16"]
    assert kb(o.affine_bytes_per_token(2 * E, 8)) == g["affine8_g64"]
    assert kb(o.affine_bytes_per_token(2 * E, 4)) == g["affine4_g64"]
    assert kb(o.affine_bytes_per_token(2 * E, 4)) == g["turboquant4_g64"]
    assert kb(o.affine_bytes_per_token(2 * E, 3, qjl_d=128)) == g["turboquant3_g64_qjl"]
    # a 64-long norm vector would not reproduce the row: the sketch costs
    # d/8 + 2 bytes per 128-long key vector
    assert kb(o.affine_bytes_per_token(2 * E, 3, qjl_d=64)) != g["turboquant3_g64_qjl"]
    gb2k = _gold("kv_bytes_per_token.json")["kv_gb_at_2k"]
    assert round(2048 * o.affine_bytes_per_token(2 * E, 4) / 1e9, 3) == gb2k["affine4_g64"]
    assert round(2048 * o.affine_bytes_per_token(2 * E, 4, qjl_d=128) / 1e9, 3) == gb2k["affine4_g64_qjl"]
    # this library's records: d=128, K3/V4, fp16 norms = 48+2+64+2 bytes
    assert o.tq_bytes_per_token(128, 3, 4, 2, False) == 116
    assert o.tq_bytes_per_token(128, 3, 4, 2, True) == 134
    assert o.tq_bytes_per_token(256, 2, 2, 2, False) == 132
