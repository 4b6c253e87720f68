"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each mutant below is a copy of one oracle function with one plausible
mistake: a flipped sign or swapped coefficient, a dropped term, a missing
square, one iteration too few, no transpose back, the spectral instead of
the Frobenius norm, no eps, a wrong momentum or Nesterov recurrence, a
wrong update sign, an ignored per-matrix scale, weight decay applied
to the new weights, a QK-Clip that scales by tau/S instead of its root,
scales column blocks, or clips every head, diagnostics that report the
direction's RMS as the update's, the old weights' RMS, the squared
momentum norm or swapped non-finite flags, or a step that orthogonalises
the gradient instead of the momentum.  With the mutant patched into ``oracle.muon_oracle``,
the pins of ``test_oracle_pins`` run again, and at least one of them must
fail.  The unpatched oracle passes every one of them.

Two changes are deliberately not mutants, because they are not mistakes.
Working on the larger Gram side gives the same matrix function, since
NS(M^T) = NS(M)^T. Forming ``X (X^T X)`` instead of ``(X X^T) X`` is the
same product.
"""
import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import muon_oracle as orc

A0, B0, C0 = orc.NS_COEFFS
ORIG_DIAGNOSTICS = orc.diagnostics


def _ns(update, steps_adj=0, back=True, normalize=None):
    """A Newton-Schulz copy whose iteration body is ``update(X)``."""

    def ns(M, steps=5, eps=1e-7, coeffs=orc.NS_COEFFS):
        X = (normalize or orc.frobenius_normalize)(M, eps)
        tr = X.shape[0] > X.shape[1]
        if tr:
            X = X.T.copy()
        for _ in range(max(0, steps + steps_adj)):
            X = update(X)
        return X.T.copy() if (tr and back) else X

    return ns


def _step(a, b, c, square=True):
    def update(X):
        A = X @ X.T
        P = b * A + c * (A @ A if square else A)
        return a * X + P @ X

    return update


def _spectral(M, eps=1e-7):
    M = np.asarray(M, dtype=np.float64)
    return M / (np.linalg.norm(M, 2) + eps)


def _no_eps(M, eps=1e-7):
    M = np.asarray(M, dtype=np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return M / np.sqrt(np.sum(M * M))


def _momentum(kind):
    def momentum(B, G, mu, nesterov=False):
        B = np.asarray(B, dtype=np.float64)
        G = np.asarray(G, dtype=np.float64)
        if kind == "mu_on_gradient":
            B_new = B + mu * G
        else:
            B_new = mu * B + G
        if nesterov:
            M = G + mu * B if kind == "nesterov_old_buffer" else G + mu * B_new
        else:
            M = B_new
        return B_new, M

    return momentum


def _update(kind):
    def apply_update(W, O, lr, scale=1.0, weight_decay=0.0):
        W = np.asarray(W, dtype=np.float64)
        O = np.asarray(O, dtype=np.float64)
        if kind == "sign":
            return W + lr * (weight_decay * W + scale * O)
        if kind == "scale_ignored":
            return W - lr * (weight_decay * W + O)
        # decay applied to the weights after the step
        return (W - lr * scale * O) * (1.0 - lr * weight_decay)

    return apply_update


def _diagnostics(kind):
    def diagnostics(W_old, W_new, M, O):
        d = ORIG_DIAGNOSTICS(W_old, W_new, M, O)
        root_n = np.sqrt(float(np.asarray(W_new).size))
        if kind == "update from direction":
            d["update_rms"] = d["direction_rms"]
        elif kind == "old weights":
            d["weight_rms"] = float(np.linalg.norm(np.asarray(W_old, np.float64)) / root_n)
        elif kind == "squared norm":
            d["momentum_norm"] = d["momentum_norm"] ** 2
        elif kind == "flags swapped":
            f = d["nonfinite"]
            d["nonfinite"] = ((f & 1) << 1) | ((f >> 1) & 1)
        return d

    return diagnostics


def _step_on_gradient(W, G, B, mu, lr, scale=1.0, ns_steps=5, nesterov=False, eps=1e-7, weight_decay=0.0):
    B_new, _ = orc.momentum(B, G, mu, nesterov)
    O = orc.newton_schulz(np.asarray(G, np.float64), ns_steps, eps)
    return orc.apply_update(W, O, lr, scale, weight_decay), B_new, O


def _qk_clip(kind):
    def qk_clip(W, head_dim, max_logits, tau):
        W = np.array(W, dtype=np.float64)
        for h, s in enumerate(np.asarray(max_logits, dtype=np.float64)):
            if kind == "every head" or s > tau:
                f = tau / s if kind == "no root" else np.sqrt(tau / s)
                if kind == "columns":
                    W[:, h * head_dim:(h + 1) * head_dim] *= f
                else:
                    W[h * head_dim:(h + 1) * head_dim] *= f
        return W

    return qk_clip


MUTANTS = {
    "b sign flipped": ("newton_schulz", _ns(_step(A0, -B0, C0))),
    "a and c swapped": ("newton_schulz", _ns(_step(C0, B0, A0))),
    "c term dropped": ("newton_schulz", _ns(_step(A0, B0, 0.0))),
    "a X term dropped": ("newton_schulz", _ns(_step(0.0, B0, C0))),
    "A instead of A A": ("newton_schulz", _ns(_step(A0, B0, C0, square=False))),
    "one iteration too few": ("newton_schulz", _ns(_step(A0, B0, C0), steps_adj=-1)),
    "no transpose back": ("newton_schulz", _ns(_step(A0, B0, C0), back=False)),
    "spectral norm": ("frobenius_normalize", _spectral),
    "no eps": ("frobenius_normalize", _no_eps),
    "momentum scales the gradient": ("momentum", _momentum("mu_on_gradient")),
    "Nesterov on the old buffer": ("momentum", _momentum("nesterov_old_buffer")),
    "update sign": ("apply_update", _update("sign")),
    "scale ignored": ("apply_update", _update("scale_ignored")),
    "decay on the new weights": ("apply_update", _update("decay_after")),
    "QK-Clip factor without the root": ("qk_clip", _qk_clip("no root")),
    "QK-Clip on column blocks": ("qk_clip", _qk_clip("columns")),
    "QK-Clip on every head": ("qk_clip", _qk_clip("every head")),
    "update RMS from the direction": ("diagnostics", _diagnostics("update from direction")),
    "weight RMS of the old weights": ("diagnostics", _diagnostics("old weights")),
    "squared momentum norm": ("diagnostics", _diagnostics("squared norm")),
    "non-finite flags swapped": ("diagnostics", _diagnostics("flags swapped")),
    "direction from the gradient": ("muon_step", _step_on_gradient),
}


def _pin_calls():
    calls = [(pins.test_default_step_count_is_five, {})]
    for shape in pins.SHAPES:
        for steps in (1, 5):
            calls.append((pins.test_ns_equals_svd_closed_form, dict(shape=shape, scale=1.0, steps=steps)))
    calls += [
        (pins.test_eps_is_part_of_the_normalisation, {}),
        (pins.test_normalisation_is_frobenius_not_spectral, {}),
        (pins.test_band_after_five_steps, {}),
        (pins.test_rank_one, {}),
        (pins.test_scaled_orthogonal, {}),
        (pins.test_one_by_one, {}),
        (pins.test_zero_matrix, {}),
        (pins.test_zero_steps_is_normalisation, {}),
        (pins.test_momentum_closed_form_ten_steps, {}),
        (pins.test_nesterov_input_closed_form, {}),
        (pins.test_update_is_linear_in_direction, {}),
        (pins.test_weight_decay_zero_direction_shrinks_weights, {}),
        (pins.test_weight_decay_acts_on_old_weights_outside_direction, {}),
    ]
    for shape in [(9, 4), (4, 9), (12, 12)]:
        calls.append((pins.test_transpose_equivariance, dict(shape=shape)))
    for shape in [(10, 6), (6, 10), (8, 8)]:
        calls.append((pins.test_singular_vectors_preserved, dict(shape=shape)))
    for j, value in [(3, 0.688140), (5, 1.132924)]:
        calls.append((pins.test_signed_partial_permutation, dict(j=j, value=value)))
    for heads, head_dim, d_model in [(6, 4, 24), (5, 8, 16), (3, 16, 40)]:
        calls.append((pins.test_qk_clip_brings_every_clipped_head_to_tau,
                      dict(heads=heads, head_dim=head_dim, d_model=d_model)))
    calls += [(pins.test_qk_clip_threshold_above_every_head_is_identity, {}),
              (pins.test_qk_clip_power_of_four_factor, {})]
    calls += [(pins.test_step_follows_the_momentum_not_the_gradient, {}),
              (pins.test_diagnostics_rank_one_closed_form, {}),
              (pins.test_diagnostics_decay_only, {})]
    for n in (4, 9):
        calls.append((pins.test_diagnostics_scaled_orthogonal, dict(n=n)))
    for bad, where, flags in [(np.nan, "G", 3), (np.nan, "W", 2)]:
        calls.append((pins.test_diagnostics_nonfinite_flags, dict(bad=bad, where=where, flags=flags)))
    return calls


def _failing_pins():
    failed = []
    for fn, kw in _pin_calls():
        try:
            fn(**kw)
        except Exception:  # an assertion, or a shape error from the mutant
            failed.append(f"{fn.__name__}({kw})")
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, mutant = MUTANTS[name]
    monkeypatch.setattr(orc, attr, mutant)
    failed = _failing_pins()
    assert failed, f"no pin catches the planted mistake '{name}'"
