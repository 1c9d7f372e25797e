"""CPU checks of the test helpers that stand between the GPU and the oracle:
the matrix-core model used to attribute outputs outside the stated tolerance
(tests/parity.py HwModel), against the oracle and the truncation bound."""
import numpy as np

from parity import HwModel, hw_bound, model_fprop, model_wgrad, stated_bound, ulp_bf16

T = 128
SMALL_INT = np.array([0x00, 0x80, 0x38, 0xB8, 0x40, 0xC0, 0x44, 0xC4, 0x48, 0xC8], np.uint8)   # 0, +-1 .. +-4


def test_model_exact_window_equals_oracle(orc):
    """Small-integer products never leave the 13-bit window: the model is the
    exact block-scaled sum, i.e. the oracle."""
    g = np.random.default_rng(1)
    M, N, K = 6, 5, 384
    qx = SMALL_INT[g.integers(0, SMALL_INT.size, (M, K))]
    qwT = SMALL_INT[g.integers(0, SMALL_INT.size, (N, K))]
    sx = np.exp(g.uniform(-3, 3, (K // T, M))).astype(np.float32)
    sw = np.exp(g.uniform(-3, 3, (K // T, 1))).astype(np.float32)       # one 128-wide weight tile
    qwT = np.concatenate([qwT, np.zeros((T - N, K), np.uint8)])
    r, _ = orc.gemm_fprop(qx, sx, qwT, sw, cols=np.arange(N))
    m = model_fprop(qx, sx, qwT, sw, cols=np.arange(N))
    for i in range(M):
        for j in range(N):
            assert m(i, j) == r[i, j]


def test_model_within_truncation_bound_and_below_exact_magnitude(orc):
    """On codes with a wide exponent spread the model differs from the oracle by
    at most the truncation bound; with every product positive, truncation
    toward zero can only lower the sum."""
    g = np.random.default_rng(2)
    K, n = 256, 12
    A = g.integers(0, 0x7F, (n, K)).astype(np.uint8)        # positive codes, no NaN
    B = g.integers(0, 0x7F, (n, K)).astype(np.uint8)
    SA = np.ones((n, K // T), np.float32)
    SB = np.ones((n, K // T), np.float32)
    bound = hw_bound(A, B, SA, SB, K)
    m = HwModel(A, B, SA, SB, K)
    for i in range(n):
        r, _ = orc.gemm_wgrad(A[i:i + 1], np.ones((2, 1), np.float32), B[i:i + 1], np.ones((2, 1), np.float32), K)
        v = m(i, i)
        assert v <= r[0, 0] + 1e-12 * abs(r[0, 0])          # all products positive: truncation only lowers
        assert r[0, 0] - v <= bound[i, i] * (1 + 1e-12)
    assert np.any(bound > 0)


def test_model_wgrad_selection_matches_direct(orc):
    g = np.random.default_rng(3)
    K, N, M = 256, 128, 200
    Mp = 256
    qxT = g.integers(0, 0x7E, (K, Mp)).astype(np.uint8)
    qdyT = g.integers(0, 0x7E, (N, Mp)).astype(np.uint8)
    qxT[:, M:] = 0
    qdyT[:, M:] = 0
    sxT = np.exp(g.uniform(-2, 2, (2, K))).astype(np.float32)
    sdyT = np.exp(g.uniform(-2, 2, (2, N))).astype(np.float32)
    rows, cols = np.array([0, 77, 255]), np.array([5, 127])
    m = model_wgrad(qxT, sxT, qdyT, sdyT, M, rows, cols)
    full = HwModel(qxT, qdyT, sxT[:, :].T, sdyT[:, :].T, M)
    for a, i in enumerate(rows):
        for b, j in enumerate(cols):
            assert m(a, b) == full(i, j)


def test_stated_bound_and_ulp():
    assert ulp_bf16(1.0) == 2.0 ** -7 and ulp_bf16(1.5) == 2.0 ** -7 and ulp_bf16(2.0) == 2.0 ** -6
    assert ulp_bf16(0.0) == 2.0 ** -133
    r, aabs = np.array([1.0, 0.0, -3e-3]), np.array([10.0, 10.0, 10.0])
    t = stated_bound(r, aabs, False)
    assert np.allclose(t, [1e-3, 1e-4, 1e-4])
    tb = stated_bound(r, aabs, True)
    assert np.allclose(tb - t, ulp_bf16(r))
