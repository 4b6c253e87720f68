"""Bit-exact checks of the index logic (shape, transpose, padding, grouping,
per-matrix pointers and scales) and of determinism, through the C ABI.

Fingerprint inputs are chosen so every value on the path is exact in float32
and bf16: G has +-1 at 4^j distinct positions, W = B = 0, eps = 0 and no
Newton-Schulz step, so ||M||_F = 2^j, O = M / 2^j and
W' = -lr * scale * O are powers of two.  Any misplaced, transposed or
dropped element changes a bit.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import muon_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import matrix_muon_step_amd as m

    m.lib()
    return m


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


FINGER_SHAPES = [(1, 1, 0), (17, 33, 2), (33, 17, 2), (768, 3072, 5), (3072, 768, 5),
                 (129, 130, 3), (130, 129, 3), (1, 200, 2), (200, 1, 2), (256, 256, 4)]


def test_fingerprint_grouped_bit_exact(mm):
    print("[case] fingerprint grouped", flush=True)
    lr = 2.0 ** -4
    mats, refs = [], []
    for i, (r, c, j) in enumerate(FINGER_SHAPES):
        G = synth.sparse_signs(r, c, 4 ** j, [60, i])
        scale = 2.0 ** -(i % 4)
        W = torch.zeros(r, c, device="cuda")
        B = torch.zeros(r, c, device="cuda")
        mats.append((W, dev(G), B, scale))
        Wr, Br, _ = orc.muon_step(np.zeros((r, c)), G, np.zeros((r, c)), mu=0.95, lr=lr, scale=scale,
                                  ns_steps=0, eps=0.0)
        refs.append((Wr.astype(np.float32), Br.astype(np.float32)))
    mm.muon_step(mats, mu=0.95, lr=lr, ns_steps=0, eps=0.0)
    torch.cuda.synchronize()
    for (W, _, B, _), (Wr, Br), shp in zip(mats, refs, FINGER_SHAPES):
        assert np.array_equal(W.cpu().numpy().view(np.uint32), Wr.view(np.uint32)), shp
        assert np.array_equal(B.cpu().numpy().view(np.uint32), Br.view(np.uint32)), shp


def test_partial_permutation_five_steps(mm):
    """Support and signs exact; every nonzero magnitude bit-identical to the
    others; the common value within 2e-2 of p^5(2^-j) and equal to the
    precision scheme's scalar value."""
    print("[case] partial permutation", flush=True)
    cases = [(300, 200, 3), (200, 300, 3), (1100, 1030, 5)]
    Ms = [synth.signed_partial_permutation(r, c, 4 ** j, [61, r, c]) for r, c, j in cases]
    Os = mm.muon_orthogonalize([dev(M) for M in Ms], ns_steps=5, eps=0.0)
    torch.cuda.synchronize()
    _, plans = mm.muon_plan_query([(r, c) for r, c, _ in cases])
    for (r, c, j), M, O, pl in zip(cases, Ms, Os, plans):
        On = O.cpu().numpy()
        ref = orc.newton_schulz(M.astype(np.float64), 5, eps=0.0)
        assert np.array_equal(np.sign(On), np.sign(ref))
        mags = np.abs(On[M != 0])
        assert np.all(mags.view(np.uint32) == mags.view(np.uint32)[0])
        expect = np.abs(ref[M != 0][0])
        assert abs(mags[0] - expect) <= 2e-2 * expect
        assert mags[0] == scheme_scalar(2.0 ** -j, 5, fused=bool(pl["fused_update"]))


# Maximum shapes the library accepts (MUON_MAX_GRAM x MUON_MAX_DIM, both
# orientations) and the edges of the float32 small path at the maximum long
# side.  The matrices are built on the GPU from the generator's entries.
MAX_SHAPES = [(16384, 65536, 7), (65536, 16384, 7), (64, 65536, 3), (65, 65536, 3), (1, 65536, 0)]


@pytest.mark.parametrize("shape", MAX_SHAPES)
def test_partial_permutation_maximum_sizes(mm, shape):
    """The partial-permutation check at the largest supported shapes: support
    and signs exact, every nonzero magnitude bit-identical and equal to the
    precision scheme's scalar value (float32 small path: within 1e-5 of
    p^5(2^-j), its own rounding), no other element nonzero."""
    r, c, j = shape
    print(f"[case] partial permutation {r}x{c}, 4^{j} entries", flush=True)
    ri, ci, si = synth.signed_partial_permutation_entries(r, c, 4 ** j, [62, r, c])
    M = torch.zeros(r, c, dtype=torch.float32, device="cuda")
    rt = torch.from_numpy(ri).cuda()
    ct = torch.from_numpy(ci).cuda()
    M[rt, ct] = torch.from_numpy(si.astype(np.float32)).cuda()
    (O,) = mm.muon_orthogonalize([M], ns_steps=5, eps=0.0)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(O)) == 4 ** j
    vals = O[rt, ct].cpu().numpy()
    assert np.array_equal(np.sign(vals), si.astype(np.float32))
    mags = np.abs(vals)
    assert np.all(mags.view(np.uint32) == mags.view(np.uint32)[0])
    _, plans = mm.muon_plan_query([(r, c)])
    if plans[0]["tile"]:
        assert mags[0] == scheme_scalar(2.0 ** -j, 5, fused=bool(plans[0]["fused_update"]))
    else:
        x = 2.0 ** -j
        for _ in range(5):
            x = 3.4445 * x - 4.7750 * x ** 3 + 2.0315 * x ** 5
        assert abs(mags[0] - x) <= 1e-5 * x
    del M, O
    torch.cuda.empty_cache()


def _bf16(x):
    return np.float32(torch.tensor(float(x), dtype=torch.float32).to(torch.bfloat16).float().item())


def scheme_scalar(x0, steps, fused=False):
    """The iteration on one singular value in the library's stated precision
    scheme: iterate carried as a bf16 pair, A and P rounded to bf16, float32
    accumulation and epilogues (each a*b+c rounded once).  On an isolated
    singular value every product is exact, so the GPU must match this bit
    for bit.  The result is the final pair's sum, or with the fused update
    the last iteration's float32 value itself."""
    f = np.float32
    a, b, c = f(3.4445), f(-4.7750), f(2.0315)
    x = f(x0)
    xh = _bf16(x)
    xl = _bf16(f(x - xh))
    for _ in range(steps):
        A = _bf16(f(xh * xh))
        P = _bf16(f(np.float64(c) * np.float64(f(A * A)) + np.float64(f(b * A))))
        xn = f(np.float64(a) * np.float64(f(xh + xl)) + np.float64(f(P * xh)))
        xh = _bf16(xn)
        xl = _bf16(f(xn - xh))
    return xn if fused else f(xh + xl)


def test_grouped_equals_one_by_one(mm):
    print("[case] grouped == single", flush=True)
    w = synth.WORKLOADS["gpt2_small"]
    idx = [0, 1, 4, 5, 6, 10, 11]
    host = [synth.numpy_matrix(w, i, 0) for i in idx]
    grouped = [(dev(h["W0"]), dev(h["G"]), dev(h["B0"]), 1.0) for h in host]
    single = [(dev(h["W0"]), dev(h["G"]), dev(h["B0"]), 1.0) for h in host]
    mm.muon_step(grouped)
    for mt in single:
        mm.muon_step([mt])
    torch.cuda.synchronize()
    for a, b in zip(grouped, single):
        assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])


def test_repeat_runs_identical_and_resume(mm):
    """Same inputs twice give identical bits; 4 steps == 2 steps + host round
    trip of (W, B) + 2 steps."""
    print("[case] determinism / resume", flush=True)
    w = synth.WORKLOADS["gpt2s_fc_10step"]
    h = synth.numpy_matrix(w, 0, 0)
    Gs = [dev(synth.numpy_gradient(768, 3072, 16, 0.1, "f32", [1, 0, t, 0])) for t in range(4)]
    runs = []
    for rep in range(2):
        W, B = dev(h["W0"]), dev(h["B0"])
        for t in range(4):
            if rep == 1 and t == 2:
                Wh, Bh = W.cpu().numpy().copy(), B.cpu().numpy().copy()
                W, B = dev(Wh), dev(Bh)
            mm.muon_step([(W, Gs[t], B, 1.0)])
        torch.cuda.synchronize()
        runs.append((W.cpu().numpy(), B.cpu().numpy()))
    assert np.array_equal(runs[0][0].view(np.uint32), runs[1][0].view(np.uint32))
    assert np.array_equal(runs[0][1].view(np.uint32), runs[1][1].view(np.uint32))


def test_step_and_orthogonalize_share_bits(mm):
    """muon_step's direction equals muon_orthogonalize of the updated buffer, bit for bit."""
    print("[case] step vs orthogonalize", flush=True)
    g = synth.numpy_gradient(300, 700, 8, 0.1, "f32", [62, 0, 0, 0])
    W = torch.zeros(300, 700, device="cuda")
    B = torch.zeros(300, 700, device="cuda")
    mm.muon_step([(W, dev(g), B, 1.0)], lr=1.0)
    O = mm.muon_orthogonalize([B.clone()])[0]
    torch.cuda.synchronize()
    assert torch.equal(W, -O)
