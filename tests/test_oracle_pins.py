"""Pins of the CPU oracle to mathematics (no GPU).

Each test fixes part of ``oracle.muon_oracle`` against something other than
the oracle itself: the coefficients printed on the Muon synthesis note
(page 5, section 4; ``tests/golden/ns_coefficients.txt``), the singular
value decomposition, scalar iteration of the quintic, exact special cases
and closed forms.  A dropped term, a wrong sign or coefficient, a missing
transpose, the wrong norm or a wrong momentum recurrence fails at least one.
"""
import numpy as np
import pytest

from conftest import load_golden_coefficients
from oracle import muon_oracle as orc
from synth import signed_partial_permutation

GOLD = load_golden_coefficients()
A, B, C = GOLD["a"], GOLD["b"], GOLD["c"]
EPS = 1e-7


def p(x):
    """The scalar quintic the iteration applies to every singular value."""
    return A * x + B * x ** 3 + C * x ** 5


def p_iter(x, k):
    for _ in range(k):
        x = p(x)
    return x


def svd_closed_form(M, steps, eps=EPS):
    """U diag(p^k(s_i / (||M||_F + eps))) V^T, via numpy's SVD."""
    U, s, Vt = np.linalg.svd(M, full_matrices=False)
    nrm = np.sqrt(np.sum(M * M))
    return (U * p_iter(s / (nrm + eps), steps)) @ Vt


def rel(a, b):
    d = np.linalg.norm(a - b)
    n = np.linalg.norm(b)
    return d / n if n > 0 else d


# ------------------------------------------------------------------ coefficients
def test_coefficients_match_page():
    assert orc.NS_COEFFS == (A, B, C)
    assert int(GOLD["steps"]) == 5


def test_default_step_count_is_five():
    rng = np.random.default_rng(7)
    M = rng.standard_normal((6, 9))
    assert np.allclose(orc.newton_schulz(M), orc.newton_schulz(M, steps=5), rtol=0, atol=0)


# ------------------------------------------------------------------ SVD closed form
SHAPES = [(1, 1), (1, 7), (7, 1), (2, 3), (3, 2), (5, 5), (8, 3), (3, 8), (17, 33), (33, 17), (16, 16)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("scale", [1e-3, 1.0, 1e3])
@pytest.mark.parametrize("steps", [0, 1, 2, 5, 6])
def test_ns_equals_svd_closed_form(shape, scale, steps):
    rng = np.random.default_rng([shape[0], shape[1], steps, int(np.log10(scale)) + 5])
    M = scale * rng.standard_normal(shape)
    O = orc.newton_schulz(M, steps)
    ref = svd_closed_form(M, steps)
    assert O.shape == M.shape
    assert rel(O, ref) <= 1e-12


def test_eps_is_part_of_the_normalisation():
    # A matrix of Frobenius norm 1e-6: eps shifts every s_i by ~9 %, far
    # outside round-off, so dropping eps (or using another) fails here.
    rng = np.random.default_rng(11)
    M = rng.standard_normal((4, 6))
    M *= 1e-6 / np.linalg.norm(M)
    O = orc.newton_schulz(M, 5)
    assert rel(O, svd_closed_form(M, 5, eps=EPS)) <= 1e-12
    assert rel(O, svd_closed_form(M, 5, eps=0.0)) > 1e-3


def test_normalisation_is_frobenius_not_spectral():
    rng = np.random.default_rng(12)
    M = rng.standard_normal((6, 10))
    X = orc.frobenius_normalize(M, 0.0)
    assert abs(np.sum(X * X) - 1.0) <= 1e-14
    X_eps = orc.frobenius_normalize(M, EPS)
    nrm = np.sqrt(np.sum(M * M))
    assert np.allclose(X_eps, M / (nrm + EPS), rtol=1e-15, atol=0)


# ------------------------------------------------------------------ invariants
@pytest.mark.parametrize("shape", [(9, 4), (4, 9), (12, 12)])
def test_transpose_equivariance(shape):
    rng = np.random.default_rng(list(shape))
    M = rng.standard_normal(shape)
    assert rel(orc.newton_schulz(M.T, 5), orc.newton_schulz(M, 5).T) <= 1e-12


@pytest.mark.parametrize("shape", [(10, 6), (6, 10), (8, 8)])
def test_singular_vectors_preserved(shape):
    rng = np.random.default_rng([3] + list(shape))
    # Well separated singular values so the SVD basis is unique.
    k = min(shape)
    U, _ = np.linalg.qr(rng.standard_normal((shape[0], k)))
    V, _ = np.linalg.qr(rng.standard_normal((shape[1], k)))
    s = np.linspace(1.0, 0.1, k)
    M = (U * s) @ V.T
    O = orc.newton_schulz(M, 5)
    D = U.T @ O @ V
    off = D - np.diag(np.diag(D))
    assert np.max(np.abs(off)) <= 1e-12
    expect = p_iter(s / (np.sqrt(np.sum(s * s)) + EPS), 5)
    assert np.allclose(np.diag(D), expect, rtol=1e-12, atol=1e-13)


def test_band_after_five_steps():
    # p maps [0.6818, 1.2024] into itself, and every s >= 1.505e-3 enters it
    # within five steps; so every singular value of the output lies in the
    # band whenever the input's smallest normalised singular value does.
    rng = np.random.default_rng(5)
    for shape in [(32, 48), (48, 32), (40, 40)]:
        M = rng.standard_normal(shape)
        nrm = np.sqrt(np.sum(M * M))
        smin = np.linalg.svd(M, compute_uv=False).min() / nrm
        assert smin >= 1.505e-3
        sv = np.linalg.svd(orc.newton_schulz(M, 5), compute_uv=False)
        assert sv.min() >= 0.6818 - 1e-9 and sv.max() <= 1.2024 + 1e-9
    xs = np.linspace(0.6818, 1.2024, 20001)
    ys = p(xs)
    assert ys.min() >= 0.6818 - 1e-6 and ys.max() <= 1.2024


# ------------------------------------------------------------------ special cases
def test_rank_one():
    rng = np.random.default_rng(21)
    u = rng.standard_normal(13)
    v = rng.standard_normal(7)
    M = 1e3 * np.outer(u, v)
    O = orc.newton_schulz(M, 5)
    uh = u / np.linalg.norm(u)
    vh = v / np.linalg.norm(v)
    s = np.linalg.norm(M) / (np.linalg.norm(M) + EPS)
    assert rel(O, p_iter(s, 5) * np.outer(uh, vh)) <= 1e-12
    # Values of the composed polynomial at 1, for the record.
    seq = [p_iter(1.0, k) for k in range(6)]
    assert np.allclose(seq, [1.0, 0.701, 1.113620, 0.720706, 1.089974, 0.696436], atol=5e-7)


@pytest.mark.parametrize("j,value", [(3, 0.688140), (4, 1.070524), (5, 1.132924), (6, 0.902526)])
def test_signed_partial_permutation(j, value):
    # 4^j entries of +-1 in distinct rows and columns: all 4^j singular values
    # equal 1, ||M||_F = 2^j, so O = p^5(2^-j) * M exactly (up to eps).
    n = 4 ** j
    M = signed_partial_permutation(n + 3, n + 9, n, [j, 1]).astype(np.float64)
    O = orc.newton_schulz(M, 5)
    expect = p_iter(2.0 ** j / (2.0 ** j + EPS) * 2.0 ** -j, 5)
    assert abs(expect - value) <= 5e-7
    assert rel(O, expect * M) <= 1e-12
    assert np.all(O[M == 0] == 0.0)


def test_scaled_orthogonal():
    rng = np.random.default_rng(8)
    Q, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    O = orc.newton_schulz(3.0 * Q, 5)
    s = 3.0 / (3.0 * np.sqrt(6.0) + EPS)
    assert rel(O, p_iter(s, 5) * Q) <= 1e-12


def test_one_by_one():
    for x in [-2.5, 1e-4, 7.0]:
        O = orc.newton_schulz(np.array([[x]]), 5)
        assert abs(O[0, 0] - np.sign(x) * p_iter(abs(x) / (abs(x) + EPS), 5)) <= 1e-14


def test_zero_matrix():
    Z = np.zeros((5, 8))
    O = orc.newton_schulz(Z, 5)
    assert np.all(O == 0.0)
    W = np.arange(40.0).reshape(5, 8)
    W2, B2, O2 = orc.muon_step(W, Z, Z, mu=0.95, lr=0.02)
    assert np.all(W2 == W) and np.all(B2 == 0) and np.all(O2 == 0)


def test_zero_steps_is_normalisation():
    rng = np.random.default_rng(9)
    M = rng.standard_normal((5, 3))
    O = orc.newton_schulz(M, 0)
    assert np.allclose(O, M / (np.sqrt(np.sum(M * M)) + EPS), rtol=1e-15, atol=0)


# ------------------------------------------------------------------ momentum, update
def test_momentum_closed_form_ten_steps():
    rng = np.random.default_rng(10)
    mu = 0.95
    Gs = [rng.standard_normal((4, 6)) for _ in range(10)]
    Bv = np.zeros((4, 6))
    for G in Gs:
        Bv, M = orc.momentum(Bv, G, mu)
        assert M is Bv or np.array_equal(M, Bv)
    closed = sum(mu ** (len(Gs) - 1 - t) * G for t, G in enumerate(Gs))
    assert rel(Bv, closed) <= 1e-12


def test_nesterov_input_closed_form():
    rng = np.random.default_rng(13)
    mu = 0.9
    Gs = [rng.standard_normal((3, 5)) for _ in range(4)]
    Bv = np.zeros((3, 5))
    for G in Gs:
        Bv, M = orc.momentum(Bv, G, mu, nesterov=True)
    T = len(Gs)
    buf = sum(mu ** (T - 1 - t) * G for t, G in enumerate(Gs))
    assert rel(M, Gs[-1] + mu * buf) <= 1e-12
    assert rel(Bv, buf) <= 1e-12


def test_update_is_linear_in_direction():
    rng = np.random.default_rng(14)
    W = rng.standard_normal((7, 4))
    G = rng.standard_normal((7, 4))
    Bz = np.zeros((7, 4))
    W2, B2, O = orc.muon_step(W, G, Bz, mu=0.95, lr=0.02, scale=0.5)
    assert rel(W - W2, 0.02 * 0.5 * O) <= 1e-12
    # First step from a zero buffer: the buffer is the gradient itself.
    assert np.array_equal(B2, G)
    assert rel(O, svd_closed_form(G, 5)) <= 1e-12


def test_weight_decay_zero_direction_shrinks_weights():
    # Zero gradient from a zero buffer gives a zero direction (the eps-guarded
    # normalisation), so the decoupled decay alone acts: W <- (1 - lr * wd) W.
    rng = np.random.default_rng(15)
    W = rng.standard_normal((6, 9))
    Z = np.zeros((6, 9))
    W2, B2, O = orc.muon_step(W, Z, Z, mu=0.95, lr=0.1, weight_decay=0.3)
    assert not O.any() and not B2.any()
    assert rel(W2, (1.0 - 0.1 * 0.3) * W) <= 1e-15
    # lr * wd == 1 removes the weights entirely.
    W3, _, _ = orc.muon_step(W, Z, Z, mu=0.95, lr=0.5, weight_decay=2.0)
    assert np.abs(W3).max() <= 1e-15


def test_weight_decay_acts_on_old_weights_outside_direction():
    # The decay is decoupled: it shrinks the pre-step W and leaves the
    # orthogonalised direction untouched (the closed form through the SVD),
    # so a decay applied after the direction step, or fed into the momentum,
    # fails here.
    rng = np.random.default_rng(16)
    W = rng.standard_normal((5, 8))
    G = rng.standard_normal((5, 8))
    Bz = np.zeros((5, 8))
    lr, wd, s = 0.1, 0.5, 0.75
    W2, B2, O = orc.muon_step(W, G, Bz, mu=0.9, lr=lr, scale=s, weight_decay=wd)
    assert np.array_equal(B2, G)
    assert rel(O, svd_closed_form(G, 5)) <= 1e-12
    assert rel(W2, (1.0 - lr * wd) * W - lr * s * svd_closed_form(G, 5)) <= 1e-12
    # Without decay the step is the plain update.
    W0, _, _ = orc.muon_step(W, G, Bz, mu=0.9, lr=lr, scale=s, weight_decay=0.0)
    assert rel(W0, W - lr * s * svd_closed_form(G, 5)) <= 1e-12


# ------------------------------------------------------------------ the step as a whole
def test_step_follows_the_momentum_not_the_gradient():
    # With a zero gradient the buffer still drives the step: B' = mu B and
    # M = B', so for a rank-one B = s u v^T the direction is
    # p^5(mu s / (mu s + eps)) u v^T and W' = W - lr * scale * that.  A step
    # that orthogonalised G instead of the momentum would not move W.
    rng = np.random.default_rng(16)
    u = rng.standard_normal(5)
    u /= np.linalg.norm(u)
    v = rng.standard_normal(8)
    v /= np.linalg.norm(v)
    s, mu, lr, sc = 2.0, 0.9, 0.1, 0.5
    Bm = s * np.outer(u, v)
    W = rng.standard_normal((5, 8))
    W2, B2, O = orc.muon_step(W, np.zeros((5, 8)), Bm, mu=mu, lr=lr, scale=sc)
    q = p_iter(mu * s / (mu * s + EPS), 5)
    assert np.allclose(B2, mu * Bm, rtol=0, atol=1e-15)
    assert np.allclose(O, q * np.outer(u, v), rtol=0, atol=1e-12)
    assert np.allclose(W2, W - lr * sc * q * np.outer(u, v), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ diagnostics
def test_diagnostics_rank_one_closed_form():
    # M = s u v^T: ||M||_F = s, and every singular value of the normalised
    # input is s / (s + eps), so O = p^5(s / (s + eps)) u v^T.
    rng = np.random.default_rng(17)
    u = rng.standard_normal(6)
    u /= np.linalg.norm(u)
    v = rng.standard_normal(10)
    v /= np.linalg.norm(v)
    s = 3.0
    G = s * np.outer(u, v)
    W = np.zeros((6, 10))
    lr, sc = 0.1, 0.5
    W2, B2, O, dg = orc.muon_step_diag(W, G, np.zeros((6, 10)), mu=0.9, lr=lr, scale=sc)
    q = p_iter(s / (s + EPS), 5)
    root_n = np.sqrt(60.0)
    assert abs(dg["momentum_norm"] - s) <= 1e-14 * s
    assert abs(dg["direction_rms"] - q / root_n) <= 1e-12 * q / root_n
    assert abs(dg["update_rms"] - lr * sc * q / root_n) <= 1e-12 * lr * sc * q / root_n
    assert abs(dg["weight_rms"] - lr * sc * q / root_n) <= 1e-12 * lr * sc * q / root_n
    assert dg["nonfinite"] == 0


@pytest.mark.parametrize("n", [4, 9])
def test_diagnostics_scaled_orthogonal(n):
    # M = c Q (Q orthogonal, n x n): ||M||_F = c sqrt(n); the normalised
    # singular values are all c / (c sqrt(n) + eps), so
    # ||O||_F = sqrt(n) p^5(c / (c sqrt(n) + eps)) and the RMS divides by n.
    rng = np.random.default_rng([18, n])
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    c = 0.25
    M = c * Q
    W = rng.standard_normal((n, n))
    lr, wd = 0.05, 0.2
    W2, _, O, dg = orc.muon_step_diag(W, M, np.zeros((n, n)), mu=0.5, lr=lr, weight_decay=wd)
    q = p_iter(c / (c * np.sqrt(n) + EPS), 5)
    assert abs(dg["momentum_norm"] - c * np.sqrt(n)) <= 1e-13
    assert abs(dg["direction_rms"] - q / np.sqrt(n)) <= 1e-12
    # step = -lr (wd W + O): its RMS by the same definition, with O = q Q.
    step = lr * (wd * W + q * Q)
    assert abs(dg["update_rms"] - np.linalg.norm(step) / n) <= 1e-12
    assert abs(dg["weight_rms"] - np.linalg.norm(W - step) / n) <= 1e-12


def test_diagnostics_decay_only():
    # A zero gradient: no direction, the step is the decay alone, so the
    # update RMS is lr * wd times the old weight RMS and the new weight RMS
    # is (1 - lr * wd) times it.
    rng = np.random.default_rng(19)
    W = rng.standard_normal((7, 5))
    Z = np.zeros((7, 5))
    lr, wd = 0.1, 0.3
    _, _, _, dg = orc.muon_step_diag(W, Z, Z, mu=0.95, lr=lr, weight_decay=wd)
    rms = np.sqrt(np.mean(W * W))
    assert dg["momentum_norm"] == 0.0 and dg["direction_rms"] == 0.0
    assert abs(dg["update_rms"] - lr * wd * rms) <= 1e-14
    assert abs(dg["weight_rms"] - (1 - lr * wd) * rms) <= 1e-14


@pytest.mark.parametrize("bad,where,flags", [(np.nan, "G", 3), (np.inf, "G", 3), (-np.inf, "B", 3),
                                             (np.nan, "W", 2)])
def test_diagnostics_nonfinite_flags(bad, where, flags):
    # A non-finite gradient or momentum entry makes M non-finite, and the
    # iteration spreads it to every entry of O and so of W; a non-finite
    # weight leaves M finite and shows up in W_new only.
    rng = np.random.default_rng(20)
    arrs = {k: rng.standard_normal((4, 6)) for k in ("W", "G", "B")}
    arrs[where][1, 2] = bad
    with np.errstate(invalid="ignore"):  # inf / inf in the normalisation
        W2, _, _, dg = orc.muon_step_diag(arrs["W"], arrs["G"], arrs["B"], mu=0.9, lr=0.02)
    assert dg["nonfinite"] == flags
    _, _, _, ok = orc.muon_step_diag(rng.standard_normal((4, 6)), rng.standard_normal((4, 6)),
                                     np.zeros((4, 6)), mu=0.9, lr=0.02)
    assert ok["nonfinite"] == 0


# ---------------------------------------------------------------- QK-Clip (reading R18)
def _head_max_logits(Wq, Wk, X, head_dim):
    """Per-head max attention logit of tokens X, q.k / sqrt(head_dim)."""
    H = Wq.shape[0] // head_dim
    out = np.empty(H)
    for h in range(H):
        rows = slice(h * head_dim, (h + 1) * head_dim)
        Q = X @ Wq[rows].T
        K = X @ Wk[rows].T
        out[h] = np.max(Q @ K.T) / np.sqrt(head_dim)
    return out


@pytest.mark.parametrize("heads,head_dim,d_model", [(6, 4, 24), (5, 8, 16), (3, 16, 40)])
def test_qk_clip_brings_every_clipped_head_to_tau(heads, head_dim, d_model):
    """Clipping the query and the key projection of one attention layer with
    the same per-head max logits: every head whose max logit exceeded tau
    now has max logit tau (logits are bilinear in the two projections, each
    scaled by sqrt(tau / S)); every other head keeps its rows bit for bit."""
    rng = np.random.default_rng([90, heads, head_dim])
    Wq = rng.standard_normal((heads * head_dim, d_model)) * rng.uniform(0.5, 3.0, (heads * head_dim, 1))
    Wk = rng.standard_normal((heads * head_dim, d_model))
    X = rng.standard_normal((12, d_model))
    S = _head_max_logits(Wq, Wk, X, head_dim)
    tau = float(np.median(S))
    Wq2 = orc.qk_clip(Wq, head_dim, S, tau)
    Wk2 = orc.qk_clip(Wk, head_dim, S, tau)
    S2 = _head_max_logits(Wq2, Wk2, X, head_dim)
    clipped = S > tau
    assert 0 < clipped.sum() < heads
    assert np.allclose(S2[clipped], tau, rtol=1e-12, atol=0)
    assert np.array_equal(S2[~clipped], S[~clipped])
    for h in np.flatnonzero(~clipped):
        rows = slice(h * head_dim, (h + 1) * head_dim)
        assert np.array_equal(Wq2[rows], Wq[rows]) and np.array_equal(Wk2[rows], Wk[rows])


def test_qk_clip_threshold_above_every_head_is_identity():
    rng = np.random.default_rng(91)
    W = rng.standard_normal((12, 7))
    S = np.array([1.0, 5.0, -2.0])
    assert np.array_equal(orc.qk_clip(W, 4, S, 5.0), W)


def test_qk_clip_power_of_four_factor():
    """S = tau * 4^k scales the head's rows by exactly 2^-k."""
    W = np.arange(24.0).reshape(6, 4)
    out = orc.qk_clip(W, 2, [8.0, 2.0, 128.0], 2.0)
    assert np.array_equal(out[0:2], W[0:2] / 2) and np.array_equal(out[2:4], W[2:4])
    assert np.array_equal(out[4:6], W[4:6] / 8)
