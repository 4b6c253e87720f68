"""The library's stated precision scheme evaluated on one isolated singular
value, on the CPU (test infrastructure; no GPU code, no oracle code).

When the input of the iteration is a scaled signed partial permutation
(at most one nonzero per row and column, all of magnitude x0), X X^T is
diagonal and every product the iteration forms has one nonzero term, so
each step acts on the common magnitude alone and every product is exact.
The GPU path must then reproduce this scalar recursion bit for bit.
"""
import numpy as np
import torch

A_COEF, B_COEF, C_COEF = 3.4445, -4.7750, 2.0315


def bf16(x):
    """float32 -> bf16 (round to nearest, ties to even) -> float32."""
    return np.float32(torch.tensor(float(x), dtype=torch.float32).to(torch.bfloat16).float().item())


def scheme_scalar(x0, steps, fused=False):
    """The iteration on one singular value in the library's stated precision
    scheme: iterate carried as a bf16 pair, A and P rounded to bf16, float32
    accumulation and epilogues (each a*b+c rounded once).  The result is the
    final pair's sum, or with the fused update the last iteration's float32
    value itself."""
    f = np.float32
    a, b, c = f(A_COEF), f(B_COEF), f(C_COEF)
    x = f(x0)
    xh = bf16(x)
    xl = bf16(f(x - xh))
    xn = x
    for _ in range(steps):
        A = bf16(f(xh * xh))
        P = bf16(f(np.float64(c) * np.float64(f(A * A)) + np.float64(f(b * A))))
        xn = f(np.float64(a) * np.float64(f(xh + xl)) + np.float64(f(P * xh)))
        xh = bf16(xn)
        xl = bf16(f(xn - xh))
    return xn if fused else f(xh + xl)


def p_compose(x, steps):
    """p^{o steps}(x) in float64, p(x) = a x + b x^3 + c x^5."""
    for _ in range(steps):
        x = A_COEF * x + B_COEF * x ** 3 + C_COEF * x ** 5
    return x


# Bar of the GPU magnitude against p^5(2^-j) for a signed partial
# permutation with 4^j nonzeros (the signed-permutation closed form).  Where
# the precision scheme itself, evaluated exactly (scheme_scalar), lands
# within 1e-2 of p^5(2^-j) the bar is 1e-2; at j = 3, 4 and 6 one isolated
# singular value's bf16 roundings of A and P (nothing averages over other
# singular values) put the scheme 1.06e-2, 1.03e-2 and 1.65e-2 away, and the
# bar is the Newton-Schulz bar of the whole method, 2e-2.  The GPU value is
# in every case also required to equal scheme_scalar bit for bit.
P6_GPU_BAR = {3: 2e-2, 4: 2e-2, 5: 1e-2, 6: 2e-2, 7: 1e-2, 8: 1e-2}
