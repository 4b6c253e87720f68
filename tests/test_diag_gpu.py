"""GPU parity of the per-matrix diagnostics (muon_step_diag), through the C ABI.

Bars:
  * W and B of muon_step_diag are bit-identical to muon_step's;
  * momentum_norm against the oracle's ||M||_F (float64)            <= 1e-5
  * direction_rms, update_rms, weight_rms against the same norms of
    the GPU's own O, W_new - W_old and W_new taken in float64       <= 1e-5
    (these sums run in float32 per lane on the GPU)
  * direction_rms and update_rms against the oracle's               <= 2e-2
    (the Newton-Schulz bar of the direction)
  * nonfinite flags exactly; repeated calls bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import muon_oracle as orc

pytestmark = pytest.mark.gpu

NS_TOL = 2e-2
SUM_TOL = 1e-5


@pytest.fixture(scope="module")
def mm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import matrix_muon_step_amd as m

    m.lib()
    return m


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def log_case(name):
    print(f"[case] {name}", flush=True)


def relerr(a, b):
    return abs(a - b) / abs(b) if b != 0 else abs(a)


# Fused (wide-tile last BX) and separate-update routes, both orientations,
# ragged sides, the float32 small path and a one-element matrix.
SHAPES = [(130, 1000), (1000, 132), (515, 1030), (2048, 512), (128, 128), (300, 520), (520, 300),
          (33, 17), (1, 1), (640, 1280)]


def _inputs(r, c, seed):
    rng = np.random.default_rng([seed, r, c])
    W0 = (0.02 * rng.standard_normal((r, c))).astype(np.float32)
    B0 = (0.01 * rng.standard_normal((r, c))).astype(np.float32)
    G = synth.numpy_gradient(r, c, 8, 0.1, "f32", [seed, r, c, 1])
    return W0, G, B0


def _run_pair(mm, shapes, seed, **kw):
    """One muon_step and one muon_step_diag on identical copies."""
    host = [_inputs(r, c, seed) for r, c in shapes]
    plain = [(dev(W0), dev(G), dev(B0), 1.25) for W0, G, B0 in host]
    with_d = [(dev(W0), dev(G), dev(B0), 1.25) for W0, G, B0 in host]
    mm.muon_step(plain, **kw)
    diag = mm.muon_step_diag(with_d, **kw)
    torch.cuda.synchronize()
    return host, plain, with_d, mm.diag_records(diag, len(shapes))


@pytest.mark.parametrize("shape", SHAPES)
def test_diag_matches_definitions(mm, shape):
    log_case(f"diagnostics {shape}")
    r, c = shape
    mu, lr, wd = 0.9, 0.02, 0.1
    host, plain, with_d, recs = _run_pair(mm, [shape], 81, mu=mu, lr=lr, weight_decay=wd, ns_steps=5)
    (W0, G, B0), (Wp, _, Bp, _), (Wd, _, Bd, _), rec = host[0], plain[0], with_d[0], recs[0]
    assert torch.equal(Wp.view(torch.int32), Wd.view(torch.int32))
    assert torch.equal(Bp.view(torch.int32), Bd.view(torch.int32))
    # The GPU's own direction for this momentum buffer (same kernels, same input).
    O = mm.muon_orthogonalize([Bd.clone()], ns_steps=5)[0]
    torch.cuda.synchronize()
    O64 = O.cpu().numpy().astype(np.float64)
    Wn = Wd.cpu().numpy().astype(np.float64)
    root_n = np.sqrt(float(r * c))
    assert relerr(rec["direction_rms"], np.linalg.norm(O64) / root_n) <= SUM_TOL
    assert relerr(rec["update_rms"], np.linalg.norm(Wn - W0) / root_n) <= SUM_TOL
    assert relerr(rec["weight_rms"], np.linalg.norm(Wn) / root_n) <= SUM_TOL
    assert rec["nonfinite"] == 0
    # Against the oracle.
    Wr, Br, Or, ref = orc.muon_step_diag(W0, G, B0, mu, lr, 1.25, 5, weight_decay=wd)
    assert relerr(rec["momentum_norm"], ref["momentum_norm"]) <= SUM_TOL
    assert relerr(rec["direction_rms"], ref["direction_rms"]) <= NS_TOL
    assert relerr(rec["update_rms"], ref["update_rms"]) <= NS_TOL
    assert relerr(rec["weight_rms"], ref["weight_rms"]) <= NS_TOL


def test_diag_grouped_workload_and_repeatable(mm):
    """72 matrices of the GPT-2 small set in one call: every record against
    the oracle's momentum norm and the GPU's own W; a second identical call
    gives the same records bit for bit."""
    log_case("diagnostics gpt2_small grouped")
    w = synth.WORKLOADS["gpt2_small"]
    host = [synth.numpy_matrix(w, i, 0) for i in range(len(w.matrices))]
    runs = []
    for rep in range(2):
        mats = [(dev(h["W0"]), dev(h["G"]), dev(h["B0"]), w.scale) for h in host]
        diag = mm.muon_step_diag(mats, mu=w.mu, lr=w.lr, ns_steps=5, weight_decay=0.05)
        torch.cuda.synchronize()
        runs.append((mats, diag.cpu().numpy().copy()))
    assert np.array_equal(runs[0][1], runs[1][1])
    recs = mm.diag_records(runs[0][1], len(host))
    for h, (Wd, _, _, _), rec in zip(host, runs[0][0], recs):
        _, M = orc.momentum(h["B0"], h["G"], w.mu)
        assert relerr(rec["momentum_norm"], float(np.linalg.norm(M))) <= SUM_TOL
        Wn = Wd.cpu().numpy().astype(np.float64)
        root_n = np.sqrt(float(Wn.size))
        assert relerr(rec["update_rms"], np.linalg.norm(Wn - h["W0"]) / root_n) <= SUM_TOL
        assert relerr(rec["weight_rms"], np.linalg.norm(Wn) / root_n) <= SUM_TOL
        assert rec["nonfinite"] == 0


@pytest.mark.parametrize("shape", [(300, 520), (33, 17), (2048, 512)])
@pytest.mark.parametrize("where,bad,flags", [("G", float("nan"), 3), ("G", float("inf"), 3),
                                             ("W", float("nan"), 2)])
def test_diag_nonfinite_flags(mm, shape, where, bad, flags):
    log_case(f"diagnostics non-finite {where}={bad} {shape}")
    r, c = shape
    W0, G, B0 = _inputs(r, c, 82)
    (W0 if where == "W" else G)[r // 2, c // 3] = bad
    mats = [(dev(W0), dev(G), dev(B0), 1.0)]
    recs = mm.diag_records(mm.muon_step_diag(mats, ns_steps=5), 1)
    assert recs[0]["nonfinite"] == flags


def test_diag_ns_zero_and_bf16(mm):
    """ns_steps = 0 (direction = normalised momentum, separate update) and
    bfloat16 gradients."""
    log_case("diagnostics ns_steps=0, bf16")
    r, c = 256, 768
    W0, G, B0 = _inputs(r, c, 83)
    Gb = torch.from_numpy(G).to(torch.bfloat16)
    G64 = Gb.float().numpy().astype(np.float64)
    mats = [(dev(W0), Gb.cuda(), dev(B0), 1.0)]
    rec = mm.diag_records(mm.muon_step_diag(mats, ns_steps=0, lr=0.01), 1)[0]
    _, _, _, ref = orc.muon_step_diag(W0, G64, B0, 0.95, 0.01, 1.0, 0)
    for k in ("momentum_norm", "direction_rms", "update_rms", "weight_rms"):
        assert relerr(rec[k], ref[k]) <= SUM_TOL, k
