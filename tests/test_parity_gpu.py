"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Tolerances (per matrix, relative Frobenius):
  * orthogonalised direction O (bf16 matrix-core path)      <= 2e-2
  * momentum buffer B (float32)                             <= 1e-5
  * update W' against W - lr*scale*O_gpu, relative to the
    size of the step (float32 epilogue)                     <= 1e-5
Index logic (shape, transpose, padding, grouping) is checked bit for bit in
tests/test_bitexact_gpu.py.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import muon_oracle as orc

pytestmark = pytest.mark.gpu

NS_TOL = 2e-2
FP32_TOL = 1e-5


@pytest.fixture(scope="module")
def mm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import matrix_muon_step_amd as m

    m.lib()
    return m


def relfro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def g_tensor(g, g_dtype):
    if g_dtype == "bf16":
        return torch.from_numpy(g.view(np.int16)).cuda().view(torch.bfloat16)
    return dev(g)


def log_case(name):
    print(f"[case] {name}", flush=True)


# ------------------------------------------------------------------ orthogonalisation alone
ORTHO_SHAPES = [(1, 1), (1, 300), (300, 1), (17, 33), (33, 17), (128, 128), (129, 257),
                (257, 129), (256, 256), (300, 520), (520, 300), (640, 130), (768, 3072)]


@pytest.mark.parametrize("shape", ORTHO_SHAPES)
def test_orthogonalize_matches_oracle(mm, shape):
    log_case(f"ortho {shape}")
    r, c = shape
    M = synth.numpy_gradient(r, c, min(16, r, c), 0.1, "f32", [50, r, c, 0])
    O = mm.muon_orthogonalize([dev(M)], ns_steps=5)[0]
    torch.cuda.synchronize()
    ref = orc.newton_schulz(M.astype(np.float64), 5)
    err = relfro(O.cpu().numpy(), ref)
    print(f"  relFro {err:.3e}")
    assert err <= NS_TOL


@pytest.mark.parametrize("shape", [(1, 300), (2, 5), (3, 5), (5, 3), (1, 1), (40, 40), (64, 700), (700, 64),
                                   (64, 64), (7, 9000)])
def test_small_gram_path_is_float32(mm, shape):
    """m <= 64 runs the float32 iteration: far inside the bf16 tolerance even
    for flat (Gaussian) spectra, where bf16 operands would not be."""
    log_case(f"small path {shape}")
    rng = np.random.default_rng(list(shape))
    M = rng.standard_normal(shape).astype(np.float32)
    O = mm.muon_orthogonalize([dev(M)], ns_steps=5)[0]
    torch.cuda.synchronize()
    err = relfro(O.cpu().numpy(), orc.newton_schulz(M.astype(np.float64), 5))
    print(f"  relFro {err:.3e}")
    assert err <= 1e-4


@pytest.mark.parametrize("shape", [(65, 300), (300, 65), (96, 96), (128, 256), (200, 200)])
def test_flat_spectrum_bf16_path(mm, shape):
    """Gaussian matrices just above the float32 threshold: the hardest case for
    the bf16 path (singular values spread over the whole band)."""
    log_case(f"flat spectrum {shape}")
    rng = np.random.default_rng([7] + list(shape))
    M = rng.standard_normal(shape).astype(np.float32)
    O = mm.muon_orthogonalize([dev(M)], ns_steps=5)[0]
    torch.cuda.synchronize()
    err = relfro(O.cpu().numpy(), orc.newton_schulz(M.astype(np.float64), 5))
    print(f"  relFro {err:.3e}")
    assert err <= NS_TOL


@pytest.mark.parametrize("steps", [0, 1, 2, 3, 6])
def test_orthogonalize_step_counts(mm, steps):
    log_case(f"ortho steps={steps}")
    shapes = [(200, 330), (330, 200), (64, 64)]
    Ms = [synth.numpy_gradient(r, c, 8, 0.1, "f32", [51, r, c, steps]) for r, c in shapes]
    Os = mm.muon_orthogonalize([dev(M) for M in Ms], ns_steps=steps)
    torch.cuda.synchronize()
    for M, O in zip(Ms, Os):
        ref = orc.newton_schulz(M.astype(np.float64), steps)
        tol = 1e-2 if steps == 0 else NS_TOL
        assert relfro(O.cpu().numpy(), ref) <= tol


def test_orthogonalize_grouped_mixed_shapes(mm):
    log_case("ortho grouped mixed")
    shapes = [(1, 1), (5, 3), (3, 5), (128, 384), (384, 128), (250, 250), (96, 700)]
    Ms = [synth.numpy_gradient(r, c, min(4, r, c), 0.1, "f32", [52, i, 0, 0]) for i, (r, c) in enumerate(shapes)]
    Os = mm.muon_orthogonalize([dev(M) for M in Ms], ns_steps=5)
    torch.cuda.synchronize()
    for M, O in zip(Ms, Os):
        assert relfro(O.cpu().numpy(), orc.newton_schulz(M.astype(np.float64), 5)) <= NS_TOL


# ------------------------------------------------------------------ full step helpers
def run_workload(mm, w, steps=None, nesterov=False, indices=None, weight_decay=0.0):
    """Runs `steps` Muon steps of workload w on the GPU and the oracle."""
    steps = w.steps if steps is None else steps
    idx = list(range(len(w.matrices))) if indices is None else list(indices)
    host = [synth.numpy_matrix(w, i, 0) for i in idx]
    W = [dev(h["W0"]) for h in host]
    B = [dev(h["B0"]) for h in host]
    Wref = [h["W0"].astype(np.float64) for h in host]
    Bref = [h["B0"].astype(np.float64) for h in host]
    for t in range(steps):
        gs = [synth.numpy_gradient(w.matrices[i].rows, w.matrices[i].cols, w.rank, w.noise, w.g_dtype,
                                   [w.wid, i, t, 0]) for i in idx]
        G = [g_tensor(g, w.g_dtype) for g in gs]
        mm.muon_step([(W[k], G[k], B[k], w.scale) for k in range(len(idx))], mu=w.mu, lr=w.lr,
                     ns_steps=5, nesterov=nesterov, weight_decay=weight_decay)
        for k, g in enumerate(gs):
            g64 = synth.gradient_as_f64(g, w.g_dtype)
            Wref[k], Bref[k], _ = orc.muon_step(Wref[k], g64, Bref[k], w.mu, w.lr, w.scale, 5, nesterov,
                                                weight_decay=weight_decay)
    torch.cuda.synchronize()
    return host, W, B, Wref, Bref


def check_step_results(host, W, B, Wref, Bref, lr_scale):
    worst = 0.0
    for h, Wg, Bg, Wr, Br in zip(host, W, B, Wref, Bref):
        b_err = relfro(Bg.cpu().numpy(), Br)
        assert b_err <= FP32_TOL, f"momentum relFro {b_err:.3e}"
        dW = Wg.cpu().numpy().astype(np.float64) - h["W0"]
        dref = Wr - h["W0"]
        err = relfro(dW, dref)
        worst = max(worst, err)
        assert err <= NS_TOL, f"direction relFro {err:.3e}"
    print(f"  worst direction relFro {worst:.3e}")


def test_single256(mm):
    log_case("single256")
    w = synth.WORKLOADS["single256"]
    check_step_results(*run_workload(mm, w), w.lr * w.scale)


def test_single256_update_epilogue_fp32(mm):
    """W' against W - lr*scale*O computed from the GPU's own O (float32 bar)."""
    log_case("single256 update epilogue")
    w = synth.WORKLOADS["single256"]
    h = synth.numpy_matrix(w, 0, 0)
    _check_update_against_direction(mm, h["W0"], h["G"], w.mu, w.lr, 0.75)


# Shapes of both update routes: the wide-tile BX kernels write W from their
# last launch (fused), the others leave it to the separate update pass.  The
# list covers both orientations, ragged Gram sides, rows whose length is not
# a multiple of 4 (element-wise W accesses), and 160-row BX tiles that start
# at an odd multiple of 32 rows (m = 480, 800: epilogue blocks paired from
# the second one).
UPDATE_SHAPES = [(130, 1000), (1000, 132), (515, 1030), (1030, 515), (2048, 512),
                 (128, 128), (300, 520), (520, 300), (33, 17), (480, 960), (1000, 800)]


@pytest.mark.parametrize("shape", UPDATE_SHAPES)
def test_update_routes_fp32(mm, shape):
    log_case(f"update route {shape}")
    r, c = shape
    rng = np.random.default_rng([71, r, c])
    W0 = (0.02 * rng.standard_normal((r, c))).astype(np.float32)
    G = synth.numpy_gradient(r, c, 8, 0.1, "f32", [71, r, c, 1])
    _check_update_against_direction(mm, W0, G, 0.95, 0.02, 1.5)


@pytest.mark.parametrize("shape", UPDATE_SHAPES)
def test_update_routes_weight_decay_fp32(mm, shape):
    log_case(f"update route {shape}, weight decay 0.1")
    r, c = shape
    rng = np.random.default_rng([72, r, c])
    W0 = (0.02 * rng.standard_normal((r, c))).astype(np.float32)
    G = synth.numpy_gradient(r, c, 8, 0.1, "f32", [72, r, c, 1])
    _check_update_against_direction(mm, W0, G, 0.95, 0.02, 1.5, weight_decay=0.1)


@pytest.mark.parametrize("shape", [(130, 1000), (1000, 132), (2048, 512), (300, 520), (33, 17)])
def test_weight_decay_alone_bit_exact(mm, shape):
    """A zero gradient gives a zero direction, so the step is the decay alone.
    With lr * weight_decay a power of two the float32 result is the single
    rounding of W * (1 - 2^-7), which float64 holds exactly."""
    log_case(f"weight decay alone {shape}")
    r, c = shape
    rng = np.random.default_rng([73, r, c])
    W0 = rng.standard_normal((r, c)).astype(np.float32)
    Wd = dev(W0)
    Gd, Bd = torch.zeros_like(Wd), torch.zeros_like(Wd)
    mm.muon_step([(Wd, Gd, Bd, 1.0)], lr=2.0 ** -4, weight_decay=2.0 ** -3, ns_steps=5)
    torch.cuda.synchronize()
    expect = (W0.astype(np.float64) * (1.0 - 2.0 ** -7)).astype(np.float32)
    assert np.array_equal(Wd.cpu().numpy().view(np.uint32), expect.view(np.uint32))
    assert torch.count_nonzero(Bd).item() == 0


def test_weight_decay_multi_step(mm):
    log_case("gpt2s_fc 3 steps, weight decay 0.1")
    w = synth.WORKLOADS["gpt2s_fc_10step"]
    check_step_results(*run_workload(mm, w, steps=3, weight_decay=0.1), w.lr)


def _check_update_against_direction(mm, W0, G, mu, lr, scale, offset=4, weight_decay=0.0):
    """W sits inside a larger buffer (16-byte aligned, as the ABI requires)
    with guard bands on both sides that must stay untouched."""
    r, c = W0.shape
    store = torch.zeros(r * c + offset + 64, dtype=torch.float32, device="cuda")
    Wd = store[offset:offset + r * c].view(r, c)
    Wd.copy_(dev(W0))
    Gd, Bd = dev(G), torch.zeros(r, c, dtype=torch.float32, device="cuda")
    mm.muon_step([(Wd, Gd, Bd, scale)], mu=mu, lr=lr, ns_steps=5, weight_decay=weight_decay)
    O = mm.muon_orthogonalize([Bd.clone()], ns_steps=5)[0]
    torch.cuda.synchronize()
    O64 = O.cpu().numpy().astype(np.float64)
    W64 = W0.astype(np.float64)
    lwd = np.float64(np.float32(np.float32(lr) * np.float32(weight_decay)))
    expect = W64 - lwd * W64 - np.float64(np.float32(lr * scale)) * O64
    step = expect - W0
    err = np.linalg.norm(Wd.cpu().numpy() - expect) / np.linalg.norm(step)
    assert err <= FP32_TOL, err
    assert relfro(Bd.cpu().numpy(), G) == 0.0  # first step from B = 0: B = G exactly
    # nothing outside W was touched
    assert torch.count_nonzero(store[:offset]).item() == 0
    assert torch.count_nonzero(store[offset + r * c:]).item() == 0
    # and the direction itself is the oracle's, to the Newton-Schulz bar
    ref = orc.newton_schulz(G.astype(np.float64), 5)
    assert relfro(O64, ref) <= NS_TOL


def test_gpt2s_fc_ten_steps(mm):
    log_case("gpt2s_fc_10step")
    w = synth.WORKLOADS["gpt2s_fc_10step"]
    check_step_results(*run_workload(mm, w), w.lr)


def test_gpt2_small_grouped(mm):
    log_case("gpt2_small (72 matrices, one grouped launch per stage)")
    w = synth.WORKLOADS["gpt2_small"]
    check_step_results(*run_workload(mm, w), w.lr)


def test_nesterov_reading(mm):
    log_case("nesterov")
    w = synth.WORKLOADS["gpt2s_fc_10step"]
    check_step_results(*run_workload(mm, w, steps=3, nesterov=True), w.lr)


def test_bf16_gradients_small(mm):
    log_case("bf16 gradients (moe-like aspect ratios, reduced sizes)")
    w = synth.Workload(40, "moe_small", (synth.MatrixSpec(256, 896, "up"), synth.MatrixSpec(896, 256, "down"),
                                         synth.MatrixSpec(512, 1792, "dense")), 8, 0.05, "bf16", 2)
    check_step_results(*run_workload(mm, w), w.lr)


# The momentum pass works on tiles of 64 rows x 128 columns of M in M's own
# orientation (the transposed case covers 128 Gram-side by 64 long-side
# elements of X).  Shapes that end inside a tile in both directions, in both
# orientations, with rows whose length is not a multiple of 4, plus the
# float32 small-Gram path (m <= 64), for float32 and bf16 gradients, two
# steps (the second starts from a non-zero momentum buffer).
RAGGED_MOMENTUM = (synth.MatrixSpec(127, 129, "a"), synth.MatrixSpec(129, 127, "b"),
                   synth.MatrixSpec(65, 255, "c"), synth.MatrixSpec(255, 65, "d"),
                   synth.MatrixSpec(191, 1001, "e"), synth.MatrixSpec(1001, 191, "f"),
                   synth.MatrixSpec(63, 4097, "g"), synth.MatrixSpec(4097, 63, "h"))


@pytest.mark.parametrize("g_dtype", ["f32", "bf16"])
def test_momentum_tiles_ragged(mm, g_dtype):
    log_case(f"ragged momentum tiles, {g_dtype} gradients")
    w = synth.Workload(41, "ragged_momentum", RAGGED_MOMENTUM, 8, 0.1, g_dtype, 2)
    check_step_results(*run_workload(mm, w), w.lr)


@pytest.mark.parametrize("scale", [1e-18, 1e-12, 1.0, 1e10, 1e16])
@pytest.mark.parametrize("shape", [(300, 520), (520, 300)])
def test_gradient_scale_folded_and_normalised_paths(mm, shape, scale):
    """The first iteration takes the unnormalised pair when ||M||_F lies in
    [2^-50, 2^50] (scales 1e-12 .. 1e10 here, eps dominating the
    normaliser at 1e-12) and the separately normalised one outside (1e-18,
    1e16); both must match the oracle."""
    log_case(f"gradient scale {scale:g} {shape}")
    r, c = shape
    G = (scale * synth.numpy_gradient(r, c, 8, 0.1, "f32", [74, r, c, 0]).astype(np.float64)).astype(np.float32)
    W0 = np.zeros((r, c), np.float32)
    Wd, Gd, Bd = dev(W0), dev(G), torch.zeros(r, c, dtype=torch.float32, device="cuda")
    mm.muon_step([(Wd, Gd, Bd, 1.0)], mu=0.9, lr=0.5, ns_steps=5)
    torch.cuda.synchronize()
    Wref, _, _ = orc.muon_step(W0, G, np.zeros((r, c)), 0.9, 0.5)
    assert np.isfinite(Wd.cpu().numpy()).all()
    assert relfro(Wd.cpu().numpy(), Wref) <= NS_TOL


def test_many_small_matrices_grouped(mm):
    """600 matrices in one call, mostly with a Gram side <= 64 (normalised by
    the prep pass) and a few folded ones: every matrix against the oracle."""
    log_case("600 mixed matrices, one call")
    rng = np.random.default_rng(75)
    shapes = [(int(rng.integers(1, 65)), int(rng.integers(1, 300))) for _ in range(590)]
    shapes += [(int(rng.integers(65, 200)), int(rng.integers(65, 400))) for _ in range(10)]
    host, mats = [], []
    for i, (r, c) in enumerate(shapes):
        if rng.random() < 0.5:
            r, c = c, r
        g = synth.numpy_gradient(r, c, 4, 0.1, "f32", [75, i, r, c])
        host.append(g)
        mats.append((dev(np.zeros((r, c), np.float32)), dev(g), torch.zeros(r, c, device="cuda"), 1.0))
    mm.muon_step(mats, mu=0.9, lr=0.1, ns_steps=5)
    torch.cuda.synchronize()
    worst = 0.0
    for g, (Wd, _, _, _) in zip(host, mats):
        ref, _, _ = orc.muon_step(np.zeros(g.shape), g, np.zeros(g.shape), 0.9, 0.1)
        err = relfro(Wd.cpu().numpy(), ref)
        worst = max(worst, err)
        assert err <= NS_TOL, (g.shape, err)
    print(f"  worst relFro {worst:.3e}")


def test_zero_gradient_leaves_weights(mm):
    log_case("zero gradient")
    Wd = dev(np.arange(12 * 20, dtype=np.float32).reshape(12, 20) * 1e-3)
    W0 = Wd.clone()
    Gd = torch.zeros_like(Wd)
    Bd = torch.zeros_like(Wd)
    mm.muon_step([(Wd, Gd, Bd, 1.0)], ns_steps=5)
    torch.cuda.synchronize()
    assert torch.equal(Wd, W0) and torch.count_nonzero(Bd) == 0


def test_poisoned_workspace_gives_finite_results(mm):
    """Workspace pre-filled with NaN bytes: every byte the path reads is written
    first.  The 320-row BX tiles of the last three shapes end in 1, 2 and 3
    valid wave columns (the rest of the tile is padding that no result reads,
    and its waves only load)."""
    log_case("poisoned workspace")
    shapes = [(130, 260), (260, 130), (17, 33), (256, 256), (320, 1600), (1650, 320), (640, 1700)]
    mats, host = [], []
    for i, (r, c) in enumerate(shapes):
        g = synth.numpy_gradient(r, c, 4, 0.1, "f32", [53, i, 0, 0])
        W0 = np.zeros((r, c), np.float32)
        host.append((W0, g))
        mats.append((dev(W0), dev(g), torch.zeros(r, c, device="cuda"), 1.0))
    nbytes = mm.muon_workspace_bytes(mats)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    mm.muon_step(mats, workspace=ws)
    torch.cuda.synchronize()
    for (W0, g), (Wd, _, _, _) in zip(host, mats):
        Wn = Wd.cpu().numpy()
        assert np.isfinite(Wn).all()
        ref, _, _ = orc.muon_step(W0, g, np.zeros_like(g), 0.95, 0.02)
        assert relfro(Wn, ref) <= NS_TOL
