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
from scheme import P6_GPU_BAR, p_compose, scheme_scalar

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
    others; the common value equal to the precision scheme's scalar value
    and within P6_GPU_BAR[j] of p^5(2^-j)."""
    print("[case] partial permutation", flush=True)
    cases = [(300, 200, 3), (200, 300, 3), (520, 300, 4), (1100, 1030, 5)]
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
        assert abs(mags[0] - expect) <= P6_GPU_BAR[j] * expect
        assert mags[0] == scheme_scalar(2.0 ** -j, 5, fused=bool(pl["fused_update"]))


# Shapes whose last BX launch writes W itself (wide-tile kernels, update
# fused into the epilogue): both orientations of the 1.5B set's shapes, a
# square one, and ragged ones whose last tile columns are padding.
FUSED_SHAPES = [(1600, 6400, 5), (6400, 1600, 5), (1600, 1600, 5), (640, 1700, 4), (1650, 320, 4)]


@pytest.mark.parametrize("ns_steps", [1, 5])
def test_fused_update_fingerprint_bit_exact(mm, ns_steps):
    """The fused last-BX route, bit for bit, in one grouped call: G is a
    signed partial permutation with 4^j nonzeros, B = 0, W = 0 on G's
    support and random elsewhere, lr * scale a power of two.  Then O has the
    common magnitude scheme_scalar(2^-j) on the support and exact zeros off
    it, so W' = -lr*scale*O on the support and W' = W everywhere else, all
    exact; B' = G.  A misplaced, transposed or dropped write of W (X-major
    pass or X^T-major pass) changes a bit."""
    print(f"[case] fused-update fingerprint, ns_steps={ns_steps}", flush=True)
    lr = 2.0 ** -4
    mats, host = [], []
    for i, (r, c, j) in enumerate(FUSED_SHAPES):
        G = synth.signed_partial_permutation(r, c, 4 ** j, [63, i, r, c])
        rng = np.random.default_rng([63, i, 1])
        W0 = rng.standard_normal((r, c)).astype(np.float32)
        W0[G != 0] = 0.0
        scale = 2.0 ** -(i % 4)
        host.append((G, W0, scale, j))
        mats.append((dev(W0), dev(G), torch.zeros(r, c, device="cuda"), scale))
    _, plans = mm.muon_plan_query([(r, c) for r, c, _ in FUSED_SHAPES], ns_steps=ns_steps)
    assert all(p["fused_update"] for p in plans)
    mm.muon_step(mats, mu=0.95, lr=lr, ns_steps=ns_steps, eps=0.0)
    torch.cuda.synchronize()
    for (G, W0, scale, j), (W, _, B, _), shp in zip(host, mats, FUSED_SHAPES):
        mag = scheme_scalar(2.0 ** -j, ns_steps, fused=True)
        expect = W0.copy()
        expect[G != 0] = np.float32(-(lr * scale)) * mag * G[G != 0]
        assert np.array_equal(W.cpu().numpy().view(np.uint32), expect.view(np.uint32)), shp
        assert np.array_equal(B.cpu().numpy().view(np.uint32), G.view(np.uint32)), shp


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


def test_grouped_equals_one_by_one(mm):
    """All 72 matrices of the GPT-2-small set in one call (256-tile
    launches) against one call per matrix (each a small call, run on the
    128-tiles, which compute the same arithmetic): identical bits."""
    print("[case] grouped == single", flush=True)
    w = synth.WORKLOADS["gpt2_small"]
    idx = list(range(len(w.matrices)))
    _, grouped_plan = mm.muon_plan_query([(w.matrices[i].rows, w.matrices[i].cols) for i in idx])
    _, single_plan = mm.muon_plan_query([(w.matrices[0].rows, w.matrices[0].cols)])
    assert grouped_plan[0]["tile"] == 256 and single_plan[0]["tile"] == 128
    host = [synth.numpy_matrix(w, i, 0) for i in idx]
    grouped = [(dev(h["W0"]), dev(h["G"]), dev(h["B0"]), 1.0) for h in host]
    single = [(dev(h["W0"]), dev(h["G"]), dev(h["B0"]), 1.0) for h in host]
    mm.muon_step(grouped)
    for mt in single:
        mm.muon_step([mt])
    torch.cuda.synchronize()
    for a, b in zip(grouped, single):
        assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])


@pytest.mark.parametrize("count", [10, 11])
def test_descriptor_upload_paths_bit_exact(mm, count):
    """A call's descriptor table reaches the workspace as a kernel argument
    up to 3 KB (10 matrices) and by a host-to-device copy above (11): both
    grouped calls equal one call per matrix (each a 512-byte table),
    bit for bit, W and B."""
    print(f"[case] descriptor upload, {count} matrices", flush=True)
    shapes = [(96 + 32 * (i % 4), 200 + 40 * i) for i in range(count)]
    host = []
    for i, (r, c) in enumerate(shapes):
        rng = np.random.default_rng([91, i])
        host.append((0.02 * rng.standard_normal((r, c))).astype(np.float32))
    gs = [synth.numpy_gradient(r, c, 8, 0.1, "f32", [91, i, 0, 1]) for i, (r, c) in enumerate(shapes)]
    grouped = [(dev(w0), dev(g), torch.zeros(w0.shape, device="cuda"), 1.0) for w0, g in zip(host, gs)]
    single = [(dev(w0), dev(g), torch.zeros(w0.shape, device="cuda"), 1.0) for w0, g in zip(host, gs)]
    for _ in range(2):
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


def test_side_stream_auto_buffers_bit_exact(mm):
    """muon_step, muon_step_diag and muon_orthogonalize on a side stream,
    with the workspace, the outputs and the diagnostics array allocated by
    the binding, give the bits of the same calls on the current stream.
    Between the calls the current stream allocates and writes new tensors,
    which the allocator must not place in buffers the side-stream kernels
    may still read or write."""
    print("[case] side stream", flush=True)
    shapes = [(300, 700), (700, 300), (768, 3072), (40, 90)]
    gs = [dev(synth.numpy_gradient(r, c, 8, 0.1, "f32", [64, r, c, 0])) for r, c in shapes]
    ws0 = [dev((0.02 * np.random.default_rng([64, r, c]).standard_normal((r, c))).astype(np.float32))
           for r, c in shapes]

    def run(stream):
        mats = [(W.clone(), G, torch.zeros_like(W), 1.0) for W, G in zip(ws0, gs)]
        dmats = [(W.clone(), G, torch.zeros_like(W), 1.0) for W, G in zip(ws0, gs)]
        torch.cuda.synchronize()
        mm.muon_step(mats, stream=stream)
        churn = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
        diag = mm.muon_step_diag(dmats, stream=stream)
        churn += [torch.full((1 << 20,), 9.0, device="cuda") for _ in range(8)]
        Os = mm.muon_orthogonalize([G for G in gs], stream=stream)
        churn += [torch.full((1 << 22,), 5.0, device="cuda") for _ in range(4)]
        torch.cuda.synchronize()
        del churn
        return mats, dmats, diag, Os

    ref = run(None)
    side = torch.cuda.Stream()
    got = run(side)
    for (a, b) in zip(ref[0] + ref[1], got[0] + got[1]):
        assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])
    assert torch.equal(ref[2][:len(shapes)], got[2][:len(shapes)])
    for a, b in zip(ref[3], got[3]):
        assert torch.equal(a, b)
    # a raw HIP stream handle runs on that stream too
    h = run(side.cuda_stream)
    for (a, b) in zip(ref[0], h[0]):
        assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])
