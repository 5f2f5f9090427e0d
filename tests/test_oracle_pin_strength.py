"""The oracle's pins catch plausible mistakes: each test plants one mistake
in an oracle function (monkeypatched, CPU only, undone after the test) and
checks that the pin guarding that function fails."""

import math

import numpy as np
import pytest

import oracle as o
import oracle.turboquant as ot
import test_oracle_pins as pins


def _fails(pin, *args):
    with pytest.raises(AssertionError):
        pin(*args)


def test_off_by_one_causal_position_is_caught(monkeypatch):
    right = o.attend_prefill

    def one_early(q, cache, n_ctx, **kw):   # every query one position too early
        return right(q, cache, n_ctx - 1, **kw)

    monkeypatch.setattr(o, "attend_prefill", one_early)
    _fails(pins.test_prefill_rows_equal_brute_force_over_their_prefix, False)


def test_wrong_sphere_exponent_is_caught(monkeypatch):
    def density(z, d):                      # (d-2)/2 instead of (d-3)/2
        z = np.asarray(z, dtype=np.float64)
        inside = np.abs(z) < math.sqrt(d)
        return np.where(inside, np.clip(1.0 - z * z / d, 0.0, None) ** ((d - 2) / 2.0), 0.0)

    monkeypatch.setattr(o, "sphere_density", density)
    _fails(pins.test_sphere_density_has_unit_variance, 128)


def test_other_reading_of_qjl_constant_is_caught(monkeypatch):
    # sqrt(pi d / 2) in place of sqrt(pi / (2 d)): the factor grows by d
    monkeypatch.setattr(o, "QJL_CONST", math.pi * 128 * 128 / 2.0)
    _fails(pins.test_qjl_constant_gaussian_projection_unbiased)


def test_rotation_without_sign_flip_is_caught(monkeypatch):
    def no_signs(x, seed):
        x = np.asarray(x, dtype=np.float64)
        return o.fwht(x) / math.sqrt(x.shape[-1])

    monkeypatch.setattr(o, "rht", no_signs)
    _fails(pins.test_rht_is_orthogonal_and_matches_dense, 128, 0)


def test_dropped_qjl_term_is_caught(monkeypatch):
    right = ot._scores_rot

    def without_qjl(qr, kcodes, knorm, bits_k, tau, qjl=None, sphere=False):
        return right(qr, kcodes, knorm, bits_k, tau, None, sphere)

    monkeypatch.setattr(ot, "_scores_rot", without_qjl)
    _fails(pins.test_attention_matches_brute_force, 5, True)


def test_ties_going_down_are_caught(monkeypatch):
    def strict(z, thresholds):              # z > t instead of z >= t
        z = np.asarray(z, dtype=np.float64)
        return (z[..., None] > thresholds).sum(axis=-1).astype(np.uint8)

    monkeypatch.setattr(o, "quantize", strict)
    _fails(pins.test_quantize_is_nearest_centroid, 3)


def test_truncated_norm_is_caught(monkeypatch):
    def truncate(n, norm_dtype):            # round toward zero, not to nearest even
        n = np.asarray(n, dtype=np.float64)
        r = n.astype(ot._NORM_TYPES[norm_dtype]).astype(np.float64)
        down = np.nextafter(r.astype(ot._NORM_TYPES[norm_dtype]),
                            np.zeros_like(r).astype(ot._NORM_TYPES[norm_dtype]))
        return np.where(r > n, down.astype(np.float64), r)

    monkeypatch.setattr(ot, "round_norm", truncate)
    _fails(pins.test_encode_zero_vector_and_norm_rounding)


def test_msb_first_packing_is_caught(monkeypatch):
    def msb_first(codes, bits):
        codes = np.asarray(codes, dtype=np.uint8)
        d = codes.shape[-1]
        planes = (codes[..., :, None] >> np.arange(bits, dtype=np.uint8)) & 1
        stream = planes.reshape(codes.shape[:-1] + (d * bits,))
        return np.packbits(stream, axis=-1, bitorder="big")

    monkeypatch.setattr(o, "pack_codes", msb_first)
    _fails(pins.test_pack_hand_worked_examples)


def test_affine_bias_at_group_max_is_caught(monkeypatch):
    import oracle.affine as oa

    def top_bias(y, bits, group=64):                # bias = max, scale negative
        y = np.asarray(y, dtype=np.float64)
        d = y.shape[-1]
        L = (1 << bits) - 1
        yg = y.reshape(y.shape[:-1] + (d // group, group))
        hi, lo = yg.max(-1), yg.min(-1)
        s = ((lo - hi) / L).astype(np.float16).astype(np.float64)
        b = hi.astype(np.float16).astype(np.float64)
        u = (yg - b[..., None]) / np.where(s == 0, 1.0, s)[..., None]
        return np.clip(np.rint(u), 0, L).astype(np.uint8).reshape(y.shape), s, b

    monkeypatch.setattr(oa, "affine_quantize_group_rows", top_bias)
    monkeypatch.setattr(o, "affine_quantize_group_rows", top_bias)
    import test_oracle_affine_pins as ap
    _fails(ap.test_affine_code_is_nearest_level_of_stored_grid, 4)


def test_affine_query_rotated_the_wrong_way_is_caught(monkeypatch):
    import oracle.affine as oa
    monkeypatch.setattr(oa, "rht", o.rht_inverse)
    import test_oracle_affine_pins as ap
    _fails(ap.test_affine_attention_equals_dense_softmax_in_original_frame, 1)


def test_boundary_band_too_wide_is_caught(monkeypatch):
    right = o.boundary_mask

    def wide(z, thresholds, eps=1e-6):                  # eps 1e4 times too wide
        return right(z, thresholds, eps * 1e4)

    monkeypatch.setattr(o, "boundary_mask", wide)
    _fails(pins.test_boundary_mask_is_the_1e6_band_in_z_units, 3)


def test_boundary_band_relative_to_threshold_is_caught(monkeypatch):
    def relative(z, thresholds, eps=1e-6):              # eps * |t_k|: no band at t = 0
        z = np.asarray(z, dtype=np.float64)
        return (np.abs(z[..., None] - thresholds) < eps * np.abs(thresholds)).any(axis=-1)

    monkeypatch.setattr(o, "boundary_mask", relative)
    _fails(pins.test_boundary_mask_is_the_1e6_band_in_z_units, 3)


def test_boundary_band_in_rotated_units_is_caught(monkeypatch):
    def rotated_units(z, thresholds, eps=1e-6):         # |y - t/sqrt(d)| < eps, d = 128
        z = np.asarray(z, dtype=np.float64) / math.sqrt(128)
        return (np.abs(z[..., None] - thresholds / math.sqrt(128)) < eps).any(axis=-1)

    monkeypatch.setattr(o, "boundary_mask", rotated_units)
    _fails(pins.test_boundary_mask_is_the_1e6_band_in_z_units, 4)


def test_qjl_band_too_wide_is_caught(monkeypatch):
    right = o.qjl_boundary_mask

    def wide(w, rnorm_exact, rel=1e-6):
        return right(w, rnorm_exact, rel * 1e4)

    monkeypatch.setattr(o, "qjl_boundary_mask", wide)
    _fails(pins.test_qjl_boundary_mask_is_the_band_relative_to_the_residual_norm)


def test_qjl_band_not_scaled_by_residual_norm_is_caught(monkeypatch):
    def absolute(w, rnorm_exact, rel=1e-6):             # |w| < 1e-6, ignoring ||r||
        return np.abs(w) < rel

    monkeypatch.setattr(o, "qjl_boundary_mask", absolute)
    _fails(pins.test_qjl_boundary_mask_is_the_band_relative_to_the_residual_norm)
