"""Pins of the GEMM and epilogue oracle (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

import bruteforce
from oracle import bf16, gemm, mxfp4


def _random_mx(rng, rows, k, scale_lo=120, scale_hi=135):
    codes = rng.integers(0, 16, (rows, k)).astype(np.uint8)
    scales = rng.integers(scale_lo, scale_hi, (rows, k // 32)).astype(np.uint8)
    return codes, scales


def _exact_vals(codes, scales):
    """Fraction value of every element, from the hand table and 2**(s-127)."""
    tab = [Fraction(v) for v in mxfp4.E2M1_VALUES]      # exact: grid values are dyadic
    rows, k = codes.shape
    return [[tab[int(codes[r, j])] * Fraction(2) ** (int(scales[r, j // 32]) - 127)
             for j in range(k)] for r in range(rows)]


@pytest.mark.parametrize("m,n,k", [(4, 4, 32), (4, 4, 64), (4, 4, 96), (3, 5, 64), (5, 2, 96)])
def test_gemm_brute_force_small_tiles(m, n, k):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    ac, as_ = _random_mx(rng, m, k)
    bc, bs = _random_mx(rng, n, k)
    c = gemm.gemm(ac, as_, bc, bs)
    av, bv = _exact_vals(ac, as_), _exact_vals(bc, bs)
    assert c.shape == (m, n)
    for i in range(m):
        for j in range(n):
            # B is stored [N, K]: C[i, j] = sum_k A[i, k] * B[j, k]
            assert Fraction(c[i, j]) == bruteforce.dot_exact(av[i], bv[j])


def test_gemm_exact_on_representable_inputs():
    """Equal scales and grid values: every partial sum is an integer multiple
    of 0.25 * 2**(2s), so the result is exact; checked against int64 math."""
    rng = np.random.default_rng(7)
    m, n, k = 8, 8, 4096
    ac = rng.integers(0, 16, (m, k)).astype(np.uint8)
    bc = rng.integers(0, 16, (n, k)).astype(np.uint8)
    s = 125
    a_s = np.full((m, k // 32), s, np.uint8)
    b_s = np.full((n, k // 32), s, np.uint8)
    c = gemm.gemm(ac, a_s, bc, b_s)
    half_units = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)
    ia = half_units[ac]
    ib = half_units[bc]
    exact = (ia @ ib.T).astype(np.float64) * 0.25 * 2.0 ** (2 * (s - 127))
    assert np.array_equal(c, exact)


def test_bf16_rounding_hand_ties():
    one = 1.0
    assert bf16.round_bf16(one + 2.0 ** -8) == 1.0                     # tie -> even
    assert bf16.round_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6       # tie -> even (up)
    assert bf16.round_bf16(one + 2.0 ** -8 + 2.0 ** -20) == one + 2.0 ** -7
    assert bf16.to_bf16_bits(np.array([1.0, -2.0, 0.0]))[0:3].tolist() == [0x3F80, 0xC000, 0x0000]


# ----------------------------------------------------------------- RMSNorm --
def test_rmsnorm_unit_weight_rms():
    rng = np.random.default_rng(8)
    c = rng.standard_normal((16, 512)) * 3
    eps = 1e-6
    y = gemm.rmsnorm_head(c, 128, 512, np.ones(512), eps)
    heads_c = c.reshape(16, 4, 128)
    heads_y = y.reshape(16, 4, 128)
    ms = np.mean(heads_c ** 2, axis=2)
    rms_y = np.sqrt(np.mean(heads_y ** 2, axis=2))
    assert np.allclose(rms_y, np.sqrt(ms / (ms + eps)), rtol=1e-14)


def test_rmsnorm_constant_head_closed_form():
    """A constant head c gives y = c / sqrt(c^2 + eps) * w; with c^2 = eps
    the result is w / sqrt(2) in magnitude, so a dropped or misplaced eps fails."""
    eps = 1e-6
    c = np.full((2, 256), 1e-3)
    c[1] *= -1
    w = np.linspace(0.5, 1.5, 256)
    y = gemm.rmsnorm_head(c, 256, 256, w, eps)
    assert np.allclose(y[0], w / np.sqrt(2.0), rtol=1e-13)
    assert np.allclose(y[1], -w / np.sqrt(2.0), rtol=1e-13)


def test_rmsnorm_scale_invariance_and_passthrough():
    rng = np.random.default_rng(9)
    c = rng.standard_normal((4, 768))
    w = rng.uniform(0.5, 1.5, 512)
    y1 = gemm.rmsnorm_head(c, 256, 512, w, 0.0)
    y2 = gemm.rmsnorm_head(c * 37.0, 256, 512, w, 0.0)
    assert np.allclose(y1[:, :512], y2[:, :512], rtol=1e-13)
    assert np.array_equal(y1[:, 512:], c[:, 512:])           # V passthrough


def test_rmsnorm_heads_are_independent_and_weight_per_column():
    rng = np.random.default_rng(10)
    c = rng.standard_normal((3, 256))
    w = rng.uniform(0.5, 1.5, 256)
    y = gemm.rmsnorm_head(c, 128, 256, w, 1e-6)
    for h in range(2):
        sl = slice(128 * h, 128 * (h + 1))
        x = c[:, sl]
        manual = x / np.sqrt((x ** 2).sum(axis=1, keepdims=True) / 128 + 1e-6) * w[sl]
        assert np.allclose(y[:, sl], manual, rtol=1e-13)


def test_rmsnorm_head256_two_half_schedule():
    """The pages' head_dim=256 schedule (sum of squares of the first half,
    then of the second half, rstd from their sum, scale both halves) reaches
    the single-pass result."""
    rng = np.random.default_rng(11)
    c = rng.standard_normal((8, 256))
    w = rng.uniform(0.5, 1.5, 256)
    eps = 1e-6
    ss0 = (c[:, :128] ** 2).sum(axis=1)
    ss1 = (c[:, 128:] ** 2).sum(axis=1)
    rstd = 1.0 / np.sqrt((ss0 + ss1) / 256 + eps)
    two_pass = np.concatenate([c[:, :128] * rstd[:, None] * w[:128],
                               c[:, 128:] * rstd[:, None] * w[128:]], axis=1)
    assert np.allclose(gemm.rmsnorm_head(c, 256, 256, w, eps), two_pass, rtol=1e-13)


# ------------------------------------------------------------------ SwiGLU --
def test_silu_identities():
    z = np.linspace(-30, 30, 601)
    assert gemm.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(gemm.silu(z) - gemm.silu(-z), z, rtol=0, atol=1e-13)
    big = np.array([50.0, 100.0])
    assert np.allclose(gemm.silu(big) / big, 1.0, rtol=1e-15)
    assert abs(gemm.silu(np.array([-800.0]))[0]) == 0.0
    assert np.isclose(gemm.silu(np.array([1.0]))[0], 1.0 / (1.0 + np.e ** -1), rtol=1e-15)


def test_interleave_layout_small():
    pair, is_up = gemm.interleave_columns(4, 2)
    # physical order [g0 g1 u0 u1 g2 g3 u2 u3]
    assert pair.tolist() == [0, 1, 0, 1, 2, 3, 2, 3]
    assert is_up.tolist() == [False, False, True, True, False, False, True, True]
    pair, is_up = gemm.interleave_columns(3, 1)
    assert pair.tolist() == [0, 0, 1, 1, 2, 2]
    assert is_up.tolist() == [False, True] * 3


@pytest.mark.parametrize("g", [1, 2, 8, 16, 32])
def test_interleaved_swiglu_equals_split_halves(g):
    rng = np.random.default_rng(12 + g)
    k, n_half = 64, 64
    x = rng.standard_normal((5, k))
    wg = rng.standard_normal((k, n_half))
    wu = rng.standard_normal((k, n_half))
    phys = gemm.interleave_weight(wg, wu, g)
    c_phys = x @ phys
    ref = gemm.silu(x @ wg) * (x @ wu)
    # the split-halves formula of the pages on the un-permuted [gate | up] GEMM
    full = x @ np.concatenate([wg, wu], axis=1)
    halves = gemm.silu(full[:, :n_half]) * full[:, n_half:]
    assert np.allclose(ref, halves, rtol=1e-13, atol=1e-13)
    assert np.allclose(gemm.swiglu_from_interleaved(c_phys, g), halves, rtol=1e-12, atol=1e-12)


# SwiGLU -> block transform -> MXFP4 (the down projection's input, fused)

def _gate_up_without_zeros(rng, m, n):
    g = rng.standard_normal((m, n)) * 2.0
    u = rng.standard_normal((m, n)) * 2.0
    g[g == 0] = 0.5
    u[u == 0] = 0.5
    return g, u


@pytest.mark.parametrize("n_t", [1, 3])
def test_swiglu_transform_identity_is_requant(n_t):
    rng = np.random.default_rng(40 + n_t)
    g, u = _gate_up_without_zeros(rng, 6, 96)
    t = np.broadcast_to(np.eye(32), (n_t, 32, 32)).copy()
    c1, s1 = gemm.swiglu_transform_requantize(g, u, t)
    c2, s2 = mxfp4.quantize(g / (1.0 + np.exp(-g)) * u)     # SiLU(g) * u written out
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_swiglu_transform_signed_permutation():
    """A signed permutation per block moves and sign-flips the codes of h
    exactly and keeps every block scale; a transposed T, another block's T,
    or T applied to the gate or up alone would not."""
    rng = np.random.default_rng(44)
    g, u = _gate_up_without_zeros(rng, 8, 64)
    h = g / (1.0 + np.exp(-g)) * u
    t = np.zeros((2, 32, 32))
    perms, signs = [], []
    for b in range(2):
        perm = rng.permutation(32)
        sign = rng.choice([-1.0, 1.0], 32)
        t[b, perm, np.arange(32)] = sign                 # y_j = h_perm[j] * s_j
        perms.append(perm)
        signs.append(sign)
    c_t, s_t = gemm.swiglu_transform_requantize(g, u, t)
    c_h, s_h = mxfp4.quantize(h)
    assert np.array_equal(s_t, s_h)
    for b in range(2):
        src = c_h[:, 32 * b:32 * b + 32][:, perms[b]]
        flip = np.broadcast_to((signs[b] < 0).astype(np.uint8) << 3, src.shape)
        assert np.array_equal(c_t[:, 32 * b:32 * b + 32], src ^ flip)


def test_swiglu_transform_keeps_h_unrounded():
    """h just above an e2m1 rounding midpoint, by less than bf16 resolution:
    the code rounds up.  (A bf16 copy of h would sit on the midpoint and
    round to even, i.e. down.)  Block scale fixed by an element of 5.5 * 2^s."""
    s = -3
    targets = [5.5, 0.25 + 2.0 ** -12, 1.25 + 2.0 ** -10, 2.5 + 2.0 ** -9]   # scaled values q
    want = [7, 1, 3, 5]                                   # codes of 6, 0.5, 1.5, 3
    g = np.full((1, 32), 3.0)
    silu_g = 3.0 / (1.0 + np.exp(-3.0))
    q = np.full(32, 0.5)
    q[:4] = targets
    u = (q * 2.0 ** s / silu_g)[None]
    c, sc = gemm.swiglu_transform_requantize(g, u, np.eye(32)[None])
    assert sc[0, 0] == 127 + s
    assert list(c[0, :4]) == want
    # the same values rounded to bf16 first land on midpoints and round to even
    hb = bf16.round_bf16(g / (1.0 + np.exp(-g)) * u)
    cb, _ = mxfp4.quantize(hb)
    assert list(cb[0, 1:4]) == [0, 2, 4]
