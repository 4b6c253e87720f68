"""Plain float64 CPU oracle of one Muon optimizer step.

TEST INFRASTRUCTURE.  This module exists to check the GPU library; only the
tests, the smoke check and the benchmark's CPU-baseline leg may use it.  It
shares no code, constant table or helper with the GPU path, and the GPU
path never imports it.

What it computes follows "Muon: An optimizer for hidden layers in neural
networks", the synthesis note on papers.chlience.com, section 4 (the
algorithm definition): a momentum buffer accumulates the gradient, the
momentum matrix is orthogonalised by a quintic Newton-Schulz iteration
after Frobenius normalisation (working on the transpose when that makes the
Gram matrix smaller), and the weights move against the orthogonalised
direction scaled by the learning rate.

Everything is float64; inputs are widened exactly.  Every matrix product is
a plain numpy ``@``; there is no blocking, fusion or reordering.

Readings where the page is silent (all listed again in the design notes):

* Nesterov: the page says implementations often use a Nesterov-style
  momentum but gives no formula.  Default: the Newton-Schulz input is the
  momentum buffer itself.  With ``nesterov=True`` the input is
  ``G + mu * B_new``.
* The Frobenius normalisation divides by ``||M||_F + eps`` (eps = 1e-7); a
  zero matrix therefore gives a zero direction.
* Transpose exactly when rows > cols; a square matrix is not transposed.
* ``scale`` is a caller-supplied per-matrix multiplier of the learning rate
  (the "consistent update RMS" adjustment of the Moonlight results section
  has no formula on the pages).
* Weight decay: the Moonlight results section (key experiments, result 2)
  adds decoupled weight decay in the AdamW manner, without a formula.  The
  plain reading of "decoupled" is that the decay acts on the weights
  directly, outside the momentum and the orthogonalisation:
  ``W_new = W - lr * (weight_decay * W + scale * O)``, with the old W in
  both terms.  ``weight_decay = 0`` is plain Muon.

Parity pins (tests/test_oracle_pins.py) tie every function here to
mathematics rather than to itself: the SVD closed form of the iteration,
transpose equivariance, singular vectors, the polynomial band, rank-one,
partial-permutation and zero special cases, the momentum closed form and
the update's linearity; the diagnostics by rank-one and scaled-orthogonal
closed forms, the decay-only step and the non-finite cases; QK-Clip by the
max logit it leaves on every head of random attention projections.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

# Tuned quintic coefficients (a, b, c), page 5, section 4.
NS_COEFFS = (3.4445, -4.7750, 2.0315)


def momentum(B: np.ndarray, G: np.ndarray, mu: float, nesterov: bool = False
             ) -> Tuple[np.ndarray, np.ndarray]:
    """Momentum accumulation, section 4: ``B_t = mu * B_{t-1} + G_t``.

    Returns ``(B_t, M)`` where ``M`` is the matrix handed to the
    orthogonalisation: ``B_t`` itself, or ``G + mu * B_t`` for the
    Nesterov-style reading.
    """
    B = np.asarray(B, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    B_new = mu * B + G
    M = G + mu * B_new if nesterov else B_new
    return B_new, M


def frobenius_normalize(M: np.ndarray, eps: float = 1e-7) -> np.ndarray:
    """Divide by the Frobenius norm plus eps (section 4, last paragraph)."""
    M = np.asarray(M, dtype=np.float64)
    return M / (np.sqrt(np.sum(M * M)) + eps)


def newton_schulz(M: np.ndarray, steps: int = 5, eps: float = 1e-7,
                  coeffs=NS_COEFFS) -> np.ndarray:
    """Quintic Newton-Schulz orthogonalisation of one matrix (section 4).

    Normalise by the Frobenius norm, work on the transpose when the matrix
    has more rows than columns (so X X^T is the smaller Gram matrix), then
    repeat ``steps`` times

        A = X X^T
        X = a X + b A X + c A A X

    and map back to the input's orientation.  ``b A X + c A A X`` is formed
    as ``(b A + c A A) X``, which is the same polynomial.
    """
    a, b, c = coeffs
    X = frobenius_normalize(M, eps)
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = X.T.copy()
    for _ in range(steps):
        A = X @ X.T
        P = b * A + c * (A @ A)
        X = a * X + P @ X
    return X.T.copy() if transposed else X


def apply_update(W: np.ndarray, O: np.ndarray, lr: float, scale: float = 1.0,
                 weight_decay: float = 0.0) -> np.ndarray:
    """Parameter update, section 4: ``W_{t+1} = W_t - lr * scale * O_t``.

    With ``weight_decay`` (the decoupled decay of the Moonlight results,
    key experiments result 2) the step also shrinks the old weights:
    ``W_{t+1} = W_t - lr * (weight_decay * W_t + scale * O_t)``.
    """
    W = np.asarray(W, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    return W - lr * (weight_decay * W + scale * O)


def muon_step(W: np.ndarray, G: np.ndarray, B: np.ndarray, mu: float, lr: float,
              scale: float = 1.0, ns_steps: int = 5, nesterov: bool = False,
              eps: float = 1e-7, weight_decay: float = 0.0):
    """One Muon step on one matrix.  Returns ``(W_new, B_new, O)`` in float64."""
    B_new, M = momentum(B, G, mu, nesterov)
    O = newton_schulz(M, ns_steps, eps)
    return apply_update(W, O, lr, scale, weight_decay), B_new, O


def diagnostics(W_old: np.ndarray, W_new: np.ndarray, M: np.ndarray, O: np.ndarray) -> dict:
    """Per-matrix diagnostics of one step, the layer-wise quantities the
    practice checklist of the synthesis note asks a Muon run to record
    (item 4 of its local-discussion part: update RMS per matrix shape,
    weight RMS, norm dynamics), each by its plain definition with
    N = rows * cols:

    * ``momentum_norm``: ``||M||_F`` of the Newton-Schulz input;
    * ``direction_rms``: ``||O||_F / sqrt(N)``, the orthogonalised direction
      before the learning rate and scale;
    * ``update_rms``: ``||W_new - W_old||_F / sqrt(N)``, the step applied;
    * ``weight_rms``: ``||W_new||_F / sqrt(N)``;
    * ``nonfinite``: bit 0 if M holds a NaN or an infinity, bit 1 if W_new does.
    """
    W_old = np.asarray(W_old, dtype=np.float64)
    W_new = np.asarray(W_new, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    root_n = np.sqrt(float(W_new.size))
    return dict(
        momentum_norm=float(np.sqrt(np.sum(M * M))),
        direction_rms=float(np.sqrt(np.sum(O * O)) / root_n),
        update_rms=float(np.sqrt(np.sum((W_new - W_old) ** 2)) / root_n),
        weight_rms=float(np.sqrt(np.sum(W_new * W_new)) / root_n),
        nonfinite=(0 if np.isfinite(M).all() else 1) | (0 if np.isfinite(W_new).all() else 2),
    )


def muon_step_diag(W: np.ndarray, G: np.ndarray, B: np.ndarray, mu: float, lr: float,
                   scale: float = 1.0, ns_steps: int = 5, nesterov: bool = False,
                   eps: float = 1e-7, weight_decay: float = 0.0):
    """``muon_step`` plus ``diagnostics``: returns ``(W_new, B_new, O, diag)``."""
    B_new, M = momentum(B, G, mu, nesterov)
    O = newton_schulz(M, ns_steps, eps)
    W_new = apply_update(W, O, lr, scale, weight_decay)
    return W_new, B_new, O, diagnostics(W, W_new, M, O)


def qk_clip(W: np.ndarray, head_dim: int, max_logits, tau: float) -> np.ndarray:
    """QK-Clip of the Kimi K2 result (results section, result 3, of the
    synthesis note): after the Muon step, the query and key projection
    weights of every attention head whose max logit exceeds a threshold are
    rescaled to bring that logit back.  The page gives neither the rule
    nor the threshold; the reading taken (design notes, R18):

    * ``W`` is a query or key projection in the (out, in) layout, rows
      ``h * head_dim .. (h + 1) * head_dim`` belonging to head ``h``;
    * ``max_logits[h]`` is head h's max attention logit ``S_h`` and
      ``tau > 0`` the threshold;
    * a head with ``S_h > tau`` has its rows multiplied by
      ``sqrt(tau / S_h)``.  Applied to both the query and the key
      projection, every logit of the head (bilinear in the two) is
      multiplied by ``tau / S_h``, so its max becomes ``tau``; other heads
      are left as they are.
    """
    W = np.array(W, dtype=np.float64)
    for h, s in enumerate(np.asarray(max_logits, dtype=np.float64)):
        if s > tau:
            W[h * head_dim:(h + 1) * head_dim] *= np.sqrt(tau / s)
    return W
