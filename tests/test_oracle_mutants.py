"""Plant plausible mistakes in the oracle and check that its pins catch them.

Each mutant replaces one oracle function (on the CPU, in this process only)
with a version carrying one typical slip; the pins of the other test modules
are then run and at least one must fail.  This is what makes the pins a check
of the oracle rather than of themselves.
"""

import numpy as np
import pytest

import golden_io
import test_oracle_gemm as tg
import test_oracle_mxfp4 as tm
import test_oracle_qad as tq
import test_oracle_sampler as ts
import test_oracle_transform as tt
from oracle import bf16, gemm, mxfp4, qad, sampler, transform


def _pins_mxfp4():
    for blk in golden_io.mxfp4_blocks():
        tm.test_hand_worked_blocks(blk)
    tm.test_random_blocks_against_brute_force()
    tm.test_idempotent()
    tm.test_error_bound()
    tm.test_pack_roundtrip_and_order()
    tm.test_shared_exponent_edges()


def _pins_gemm():
    for args in [(4, 4, 32), (3, 5, 64)]:
        tg.test_gemm_brute_force_small_tiles(*args)
    tg.test_gemm_exact_on_representable_inputs()
    tg.test_bf16_rounding_hand_ties()
    tg.test_rmsnorm_unit_weight_rms()
    tg.test_rmsnorm_constant_head_closed_form()
    tg.test_rmsnorm_scale_invariance_and_passthrough()
    tg.test_rmsnorm_heads_are_independent_and_weight_per_column()
    tg.test_rmsnorm_head256_two_half_schedule()
    tg.test_silu_identities()
    tg.test_interleave_layout_small()
    for g in (1, 16):
        tg.test_interleaved_swiglu_equals_split_halves(g)


def _pins_fused():
    for n_t in (1, 3):
        tg.test_swiglu_transform_identity_is_requant(n_t)
    tg.test_swiglu_transform_signed_permutation()
    tg.test_swiglu_transform_keeps_h_unrounded()


def _pins_qad():
    for blk in tq.BLOCKS:
        if blk[2] != 255:
            tq.test_fake_quantize_hand_worked_blocks(blk)
    tq.test_fake_quantize_is_idempotent_and_odd()
    tq.test_fake_quantize_keeps_grid_values()
    tq.test_ste_passes_the_gradient_unchanged()


def _pins_sampler():
    for args in [(0.9, 0.7), (0.3, 0.05)]:
        ts.test_etd1_coefficients_match_the_exact_integral(*args)
    ts.test_etd1_is_exact_over_many_steps_for_a_constant_prediction()
    ts.test_etd2_equal_predictions_and_first_step_reduce_to_etd1()
    for p in (1, 2):
        ts.test_richardson_cancels_the_leading_error(p)


def _pins_transform():
    tt.test_identity_transform_gives_plain_codes()
    tt.test_signed_permutation_permutes_codes()
    tt.test_hadamard_exact_on_small_integers()
    tt.test_fold_reconstructs_product()
    tt.test_block_locality()


def _ties_up(q):
    q = np.asarray(q, dtype=np.float64)
    return sum((q >= m).astype(np.int64) for m in mxfp4.E2M1_MIDPOINTS)


def _ties_down(q):
    q = np.asarray(q, dtype=np.float64)
    return sum((q > m).astype(np.int64) for m in mxfp4.E2M1_MIDPOINTS)


def _shared_never_saturate(amax):
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(amax / 6.0))
    return np.where(amax == 0, -127, np.clip(e, -127, 127)).astype(np.int64)


def _pack_swapped(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 1::2] | (codes[:, 0::2] << 4)).astype(np.uint8)


_orig_quantize = mxfp4.quantize


def _quantize_unsigned_zero(x, return_scaled=False):
    out = _orig_quantize(x, return_scaled)
    codes = out[0]
    x = np.asarray(x, dtype=np.float64)
    codes = np.where(x == 0, 0, codes).astype(np.uint8)
    return (codes,) + tuple(out[1:])


def _dequant_wrong_block(codes, scales):
    codes = np.asarray(codes, dtype=np.int64)
    vals = mxfp4.E2M1_VALUES[codes]
    s = mxfp4.e8m0_value(scales)
    # slip: scale of block j applied to element j % nblocks instead of j // 32
    idx = np.arange(codes.shape[1]) % s.shape[1]
    return vals * s[:, idx]


def _rms_eps_outside(c, head_dim, n_norm_cols, weight, eps):
    c = np.asarray(c, dtype=np.float64)
    y = c.copy()
    m = c.shape[0]
    h = c[:, :n_norm_cols].reshape(m, -1, head_dim)
    rstd = 1.0 / (np.sqrt(np.mean(h * h, axis=2, keepdims=True)) + eps)
    y[:, :n_norm_cols] = (h * rstd * np.asarray(weight).reshape(-1, head_dim)[None]).reshape(m, -1)
    return y


def _rms_sum_not_mean(c, head_dim, n_norm_cols, weight, eps):
    c = np.asarray(c, dtype=np.float64)
    y = c.copy()
    m = c.shape[0]
    h = c[:, :n_norm_cols].reshape(m, -1, head_dim)
    rstd = 1.0 / np.sqrt(np.sum(h * h, axis=2, keepdims=True) + eps)
    y[:, :n_norm_cols] = (h * rstd * np.asarray(weight).reshape(-1, head_dim)[None]).reshape(m, -1)
    return y


def _rms_weight_per_head(c, head_dim, n_norm_cols, weight, eps):
    c = np.asarray(c, dtype=np.float64)
    y = c.copy()
    m = c.shape[0]
    h = c[:, :n_norm_cols].reshape(m, -1, head_dim)
    rstd = 1.0 / np.sqrt(np.mean(h * h, axis=2, keepdims=True) + eps)
    w = np.asarray(weight)[: h.shape[1]][None, :, None]
    y[:, :n_norm_cols] = (h * rstd * w).reshape(m, -1)
    return y


def _rms_whole_row(c, head_dim, n_norm_cols, weight, eps):
    c = np.asarray(c, dtype=np.float64)
    y = c.copy()
    x = c[:, :n_norm_cols]
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    y[:, :n_norm_cols] = x * rstd * np.asarray(weight)[None]
    return y


def _silu_sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def _swiglu_swapped(c_gate, c_up):
    return gemm.silu(c_up) * np.asarray(c_gate, dtype=np.float64)


def _interleave_flipped(n_half, group):
    p = np.arange(2 * n_half)
    pair = (p // (2 * group)) * group + p % group
    return pair, (p // group) % 2 == 0


def _transform_transposed(x, t):
    x = np.asarray(x, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    y = np.empty_like(x)
    for b in range(x.shape[1] // 32):
        tb = t[0] if t.shape[0] == 1 else t[b]
        y[:, 32 * b:32 * b + 32] = x[:, 32 * b:32 * b + 32] @ tb.T
    return y


def _fold_transposed(w, t):
    w = np.asarray(w, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    out = np.empty_like(w)
    for b in range(w.shape[0] // 32):
        tb = t[0] if t.shape[0] == 1 else t[b]
        out[32 * b:32 * b + 32] = np.linalg.solve(tb.T, w[32 * b:32 * b + 32])
    return out


def _bf16_truncate(x):
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return ((f.view(np.uint32) >> 16).astype(np.uint16))


def _fused_h_via_bf16(c_gate, c_up, t, return_scaled=False):
    h = bf16.round_bf16(gemm.swiglu(c_gate, c_up))
    return mxfp4.quantize(transform.block_transform(h, t), return_scaled=return_scaled)


def _fused_transform_on_gate(c_gate, c_up, t, return_scaled=False):
    return mxfp4.quantize(gemm.swiglu(transform.block_transform(c_gate, t), c_up), return_scaled=return_scaled)


def _fused_transform_transposed(c_gate, c_up, t, return_scaled=False):
    t = np.swapaxes(np.asarray(t, dtype=np.float64), 1, 2)
    return mxfp4.quantize(transform.block_transform(gemm.swiglu(c_gate, c_up), t), return_scaled=return_scaled)


def _fq_truncating(x):
    x = np.asarray(x, dtype=np.float64)
    codes, scales = mxfp4.quantize(x)
    q = np.abs(x) / np.repeat(mxfp4.e8m0_value(scales), 32, axis=1)
    grid = mxfp4.E2M1_MAGNITUDES
    mag = grid[np.clip(np.searchsorted(grid, q, side="right") - 1, 0, 7)]    # round toward zero
    return np.copysign(mag, x) * np.repeat(mxfp4.e8m0_value(scales), 32, axis=1)


def _ste_halved(g):
    return 0.5 * np.asarray(g, dtype=np.float64)


def _etd1_sign_as_printed(alpha_s, sigma_s, alpha_t, sigma_t):
    h = sampler.log_snr(alpha_t, sigma_t) - sampler.log_snr(alpha_s, sigma_s)
    return np.exp(h) * alpha_t / alpha_s, alpha_t * (1.0 - np.exp(h))


def _etd2_trapezoid(alpha_s, sigma_s, alpha_t, sigma_t, first_step):
    decay, coeff = sampler.etd1_coefficients(alpha_s, sigma_s, alpha_t, sigma_t)
    return (decay, coeff, 0.0) if first_step else (decay, 0.5 * coeff, 0.5 * coeff)


def _richardson_wrong_denominator(fine, coarse, scale):
    return (scale * np.asarray(fine, dtype=np.float64) - np.asarray(coarse, dtype=np.float64)) / scale


MUTANTS = [
    ("ties_round_up", mxfp4, "encode_magnitude", _ties_up, _pins_mxfp4),
    ("ties_round_down", mxfp4, "encode_magnitude", _ties_down, _pins_mxfp4),
    ("scale_emax_1", mxfp4, "E2M1_EMAX", 1, _pins_mxfp4),
    ("scale_never_saturates", mxfp4, "shared_exponent", _shared_never_saturate, _pins_mxfp4),
    ("scale_bias_126", mxfp4, "E8M0_BIAS", 126, _pins_mxfp4),
    ("nibbles_swapped", mxfp4, "pack_codes", _pack_swapped, _pins_mxfp4),
    ("negative_zero_dropped", mxfp4, "quantize", _quantize_unsigned_zero, _pins_mxfp4),
    ("dequant_wrong_block", mxfp4, "dequantize", _dequant_wrong_block, _pins_gemm),
    ("rmsnorm_eps_outside", gemm, "rmsnorm_head", _rms_eps_outside, _pins_gemm),
    ("rmsnorm_sum_not_mean", gemm, "rmsnorm_head", _rms_sum_not_mean, _pins_gemm),
    ("rmsnorm_weight_per_head", gemm, "rmsnorm_head", _rms_weight_per_head, _pins_gemm),
    ("rmsnorm_whole_row", gemm, "rmsnorm_head", _rms_whole_row, _pins_gemm),
    ("silu_is_sigmoid", gemm, "silu", _silu_sigmoid, _pins_gemm),
    ("swiglu_gate_up_swapped", gemm, "swiglu", _swiglu_swapped, _pins_gemm),
    ("interleave_parity_flipped", gemm, "interleave_columns", _interleave_flipped, _pins_gemm),
    ("transform_transposed", transform, "block_transform", _transform_transposed, _pins_transform),
    ("fold_transposed", transform, "fold_inverse", _fold_transposed, _pins_transform),
    ("bf16_truncates", bf16, "to_bf16_bits", _bf16_truncate, _pins_gemm),
    ("fused_h_rounded_to_bf16", gemm, "swiglu_transform_requantize", _fused_h_via_bf16, _pins_fused),
    ("fused_transform_on_gate", gemm, "swiglu_transform_requantize", _fused_transform_on_gate, _pins_fused),
    ("fused_transform_transposed", gemm, "swiglu_transform_requantize", _fused_transform_transposed,
     _pins_fused),
    ("fake_quant_truncates", qad, "fake_quantize", _fq_truncating, _pins_qad),
    ("ste_scales_gradient", qad, "ste_backward", _ste_halved, _pins_qad),
    ("etd1_exponent_sign_as_printed", sampler, "etd1_coefficients", _etd1_sign_as_printed, _pins_sampler),
    ("etd2_equal_weights", sampler, "etd2_coefficients", _etd2_trapezoid, _pins_sampler),
    ("richardson_divides_by_scale", sampler, "richardson_combine", _richardson_wrong_denominator, _pins_sampler),
]


@pytest.mark.parametrize("name,module,attr,replacement,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, module, attr, replacement, pins):
    monkeypatch.setattr(module, attr, replacement)
    with pytest.raises(AssertionError):
        pins()


def test_pins_pass_unmutated():
    _pins_mxfp4()
    _pins_gemm()
    _pins_transform()
    _pins_fused()
    _pins_qad()
    _pins_sampler()
