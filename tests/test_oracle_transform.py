"""Pins of the block-transform oracle (CPU only)."""

import numpy as np

from oracle import mxfp4, transform


def _sylvester_hadamard(n):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _walsh_hadamard_int(row):
    """In-place fast Walsh-Hadamard transform of a list of Python ints
    (Sylvester ordering), i.e. row @ H_32 computed with exact integers."""
    v = list(row)
    h = 1
    while h < len(v):
        for i in range(0, len(v), 2 * h):
            for j in range(i, i + h):
                a, b = v[j], v[j + h]
                v[j], v[j + h] = a + b, a - b
        h *= 2
    return v


def test_identity_transform_gives_plain_codes():
    rng = np.random.default_rng(20)
    x = rng.standard_normal((16, 256))
    t = np.broadcast_to(np.eye(32), (8, 32, 32)).copy()
    c1, s1 = transform.transform_quantize(x, t)
    c2, s2 = mxfp4.quantize(x)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_signed_permutation_permutes_codes():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((8, 64))
    x[0, :5] = 0.0
    t = np.zeros((2, 32, 32))
    perms, signs = [], []
    for b in range(2):
        perm = rng.permutation(32)
        sign = rng.choice([-1.0, 1.0], 32)
        t[b, perm, np.arange(32)] = sign            # y_j = x_perm[j] * s_j
        perms.append(perm)
        signs.append(sign)
    c_t, s_t = transform.transform_quantize(x, t)
    c_x, s_x = mxfp4.quantize(x)
    assert (x[:, :32] == 0).any()
    assert np.array_equal(s_t, s_x)                # amax unchanged
    for b in range(2):
        src = c_x[:, 32 * b:32 * b + 32][:, perms[b]]
        flip = np.broadcast_to((signs[b] < 0).astype(np.uint8) << 3, src.shape)
        # an exact zero comes out of the sum of products as +0 (IEEE: -0 + +0 = +0)
        zero = x[:, 32 * b:32 * b + 32][:, perms[b]] == 0
        expected = np.where(zero, 0, src ^ flip)
        assert np.array_equal(c_t[:, 32 * b:32 * b + 32], expected)


def test_hadamard_exact_on_small_integers():
    rng = np.random.default_rng(22)
    x = rng.integers(-8, 9, (6, 96)).astype(np.float64)
    h = _sylvester_hadamard(32).astype(np.float64)
    y = transform.block_transform(x, h[None])
    expected = np.array([sum((_walsh_hadamard_int([int(v) for v in row[32 * b:32 * b + 32]])
                              for b in range(3)), []) for row in x], dtype=np.float64)
    assert np.array_equal(y, expected)
    c1, s1 = transform.transform_quantize(x, h[None])
    c2, s2 = mxfp4.quantize(expected)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def _random_invertible(rng, n_t):
    t = np.empty((n_t, 32, 32))
    for b in range(n_t):
        q1, _ = np.linalg.qr(rng.standard_normal((32, 32)))
        q2, _ = np.linalg.qr(rng.standard_normal((32, 32)))
        t[b] = q1 @ np.diag(rng.uniform(1.0, 3.0, 32)) @ q2
    return t


def test_fold_reconstructs_product():
    rng = np.random.default_rng(23)
    k, n = 128, 48
    x = rng.standard_normal((10, k))
    w = rng.standard_normal((k, n))
    for n_t in (1, k // 32):
        t = _random_invertible(rng, n_t)
        xt = transform.block_transform(x, t)
        wf = transform.fold_inverse(w, t)
        assert np.allclose(xt @ wf, x @ w, rtol=1e-11, atol=1e-11)


def test_block_locality():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((5, 128))
    t = _random_invertible(rng, 4)
    y1 = transform.block_transform(x, t)
    t2 = t.copy()
    t2[2] = _random_invertible(rng, 1)[0]
    y2 = transform.block_transform(x, t2)
    changed = np.any(y1 != y2, axis=0)
    assert changed[64:96].all() and not changed[:64].any() and not changed[96:].any()


def test_shared_matrix_equals_repeated_per_block():
    rng = np.random.default_rng(25)
    x = rng.standard_normal((4, 96))
    t1 = _random_invertible(rng, 1)
    t3 = np.repeat(t1, 3, axis=0)
    assert np.array_equal(transform.block_transform(x, t1), transform.block_transform(x, t3))
