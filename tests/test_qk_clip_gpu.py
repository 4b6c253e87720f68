"""QK-Clip on the GPU (muon_qk_clip) against the oracle's qk_clip, through
the C ABI.  Heads whose max logit is not above tau keep their rows bit for
bit; clipped heads meet the float32 bar (each element one rounding of W
times a correctly rounded factor), and are bit-exact where the factor is a
power of two."""
import numpy as np
import pytest
import torch

from oracle import muon_oracle as orc

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-5


@pytest.fixture(scope="module")
def mm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import matrix_muon_step_amd as m

    m.lib()
    return m


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


# (rows, cols, head_dim): the 1.5B set's Q/K (25 heads of 64), GPT-2-small's
# (12 of 64), a head whose elements are not a multiple of 4 (scalar path),
# one head, one-row heads.
CLIP_SHAPES = [(1600, 1600, 64), (768, 768, 64), (96, 30, 3), (64, 100, 64), (8, 50, 1)]


def _logits(rng, heads, tau):
    S = rng.uniform(0.2, 3.0, heads) * tau
    S[0] = tau              # at the threshold: not clipped
    if heads > 3:
        S[1] = np.nan       # not clipped
        S[2] = -5.0         # not clipped
        S[3] = np.inf       # the head's rows go to zero
    return S.astype(np.float32)


def test_qk_clip_matches_oracle(mm):
    print("[case] QK-Clip vs oracle", flush=True)
    tau = 30.0
    rng = np.random.default_rng(95)
    host, mats = [], []
    # 60 matrices: two launches (48 per launch)
    for i in range(60):
        r, c, hd = CLIP_SHAPES[i % len(CLIP_SHAPES)]
        W = rng.standard_normal((r, c)).astype(np.float32)
        S = _logits(rng, r // hd, tau)
        host.append((W, hd, S))
        mats.append((dev(W), hd, dev(S)))
    mm.muon_qk_clip(mats, tau)
    torch.cuda.synchronize()
    for (W, hd, S), (Wd, _, _) in zip(host, mats):
        got = Wd.cpu().numpy()
        ref = orc.qk_clip(W, hd, S.astype(np.float64), tau)
        for h in range(W.shape[0] // hd):
            rows = slice(h * hd, (h + 1) * hd)
            if not S[h] > tau:
                assert np.array_equal(got[rows].view(np.uint32), W[rows].view(np.uint32)), (W.shape, h)
            elif np.isinf(S[h]):
                assert not np.any(got[rows])
            else:
                err = np.linalg.norm(got[rows] - ref[rows]) / np.linalg.norm(ref[rows])
                assert err <= FP32_TOL, (W.shape, h, err)


def test_qk_clip_power_of_two_factor_bit_exact(mm):
    print("[case] QK-Clip power-of-two factors", flush=True)
    tau = 3.0
    rng = np.random.default_rng(96)
    W = rng.standard_normal((1600, 1600)).astype(np.float32)
    S = (tau * 4.0 ** rng.integers(-2, 4, 25)).astype(np.float32)
    Wd = dev(W)
    mm.muon_qk_clip([(Wd, 64, dev(S))], tau)
    torch.cuda.synchronize()
    ref = orc.qk_clip(W, 64, S.astype(np.float64), tau).astype(np.float32)
    assert np.array_equal(Wd.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_step_then_clip_on_one_stream(mm):
    """The sequence a training loop runs: a Muon step on Q and K of one layer,
    then QK-Clip of both with the layer's per-head max logits, on one side
    stream; the result is the oracle's step followed by its clip."""
    print("[case] step then QK-Clip", flush=True)
    import synth
    rng = np.random.default_rng(97)
    shapes = [(768, 768), (768, 768)]
    host = []
    for i, (r, c) in enumerate(shapes):
        g = synth.numpy_gradient(r, c, 16, 0.1, "f32", [97, i, 0, 0])
        w0 = (0.02 * rng.standard_normal((r, c))).astype(np.float32)
        host.append((w0, g))
    S = np.array([0.5, 9.0, 2.0, 40.0] * 3, np.float32)
    tau = 4.0
    side = torch.cuda.Stream()
    mats = [(dev(w0), dev(g), torch.zeros(768, 768, device="cuda"), 1.0) for w0, g in host]
    Sd = dev(S)
    torch.cuda.synchronize()
    mm.muon_step(mats, stream=side)
    mm.muon_qk_clip([(mats[0][0], 64, Sd), (mats[1][0], 64, Sd)], tau, stream=side)
    side.synchronize()
    for (w0, g), (Wd, _, _, _) in zip(host, mats):
        Wr, _, _ = orc.muon_step(w0, g, np.zeros_like(g), 0.95, 0.02)
        ref = orc.qk_clip(Wr, 64, S.astype(np.float64), tau)
        got = Wd.cpu().numpy().astype(np.float64)
        # the clip is linear per row: W' - clip(W0) = -lr * clip(O), the
        # clipped direction, held to the Newton-Schulz bar
        base = orc.qk_clip(w0, 64, S.astype(np.float64), tau)
        err = np.linalg.norm((got - base) - (ref - base)) / np.linalg.norm(ref - base)
        assert err <= 2e-2, err
