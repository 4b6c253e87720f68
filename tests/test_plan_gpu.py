"""Recorded steps (muon_plan_create / muon_plan_step) against eager
muon_step calls, through the C ABI: every replay bit-identical to the eager
step on the same inputs, with the gradient rewritten in place between
replays and eager work (other steps, allocations, synchronisations) in
between."""
import numpy as np
import pytest
import torch

import synth

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


# Every route: the float32 small path, the 16x16 and the wide-tile kernels,
# both orientations, the separate and the fused update, ragged shapes.
PLAN_SHAPES = [(256, 256), (768, 3072), (3072, 768), (40, 300), (130, 1000), (1000, 132), (480, 960)]


def _grads(shapes, step):
    return [synth.numpy_gradient(r, c, 8, 0.1, "f32", [85, i, step, 0]) for i, (r, c) in enumerate(shapes)]


@pytest.mark.parametrize("weight_decay,nesterov", [(0.0, False), (0.1, True)])
def test_plan_replays_equal_eager_steps(mm, weight_decay, nesterov):
    print(f"[case] plan replays, weight_decay={weight_decay} nesterov={nesterov}", flush=True)
    shapes = PLAN_SHAPES
    w0 = [(0.02 * np.random.default_rng([85, i]).standard_normal(s)).astype(np.float32) for i, s in enumerate(shapes)]
    kw = dict(mu=0.9, lr=0.03, ns_steps=5, nesterov=nesterov, weight_decay=weight_decay)
    # eager reference
    ref = [(dev(w), torch.zeros(s, device="cuda"), torch.zeros(s, device="cuda")) for w, s in zip(w0, shapes)]
    # recorded plan on its own buffers
    Wp = [dev(w) for w in w0]
    Gp = [torch.zeros(s, device="cuda") for s in shapes]
    Bp = [torch.zeros(s, device="cuda") for s in shapes]
    plan = mm.muon_plan_create([(W, G, B, 1.0 + 0.5 * i) for i, (W, G, B) in enumerate(zip(Wp, Gp, Bp))], **kw)
    torch.cuda.synchronize()
    for step in range(4):
        gs = _grads(shapes, step)
        for (W, G, B), g in zip(ref, gs):
            G.copy_(dev(g))
        mm.muon_step([(W, G, B, 1.0 + 0.5 * i) for i, (W, G, B) in enumerate(ref)], **kw)
        for G, g in zip(Gp, gs):
            G.copy_(dev(g))
        plan.step()
        junk = torch.randn(1 << 20, device="cuda") * 3.0   # eager work between replays
        torch.cuda.synchronize()
        del junk
        for i, ((W, _, B), Wq, Bq) in enumerate(zip(ref, Wp, Bp)):
            assert torch.equal(W, Wq), (step, shapes[i])
            assert torch.equal(B, Bq), (step, shapes[i])
    plan.close()


def test_two_plans_interleaved_on_a_side_stream(mm):
    """Two plans with separate buffers, replayed alternately on a side
    stream: each matches its own eager sequence."""
    print("[case] two plans, side stream", flush=True)
    side = torch.cuda.Stream()
    sets = [[(512, 640)], [(320, 1600), (1600, 320)]]
    plans, bufs, refs = [], [], []
    for k, shapes in enumerate(sets):
        w0 = [(0.02 * np.random.default_rng([86, k, i]).standard_normal(s)).astype(np.float32)
              for i, s in enumerate(shapes)]
        b = [(dev(w), torch.zeros(s, device="cuda"), torch.zeros(s, device="cuda")) for w, s in zip(w0, shapes)]
        r = [(dev(w), torch.zeros(s, device="cuda"), torch.zeros(s, device="cuda")) for w, s in zip(w0, shapes)]
        torch.cuda.synchronize()
        plans.append(mm.muon_plan_create([(W, G, B, 1.0) for W, G, B in b], stream=side))
        bufs.append(b)
        refs.append(r)
    for step in range(3):
        for k, shapes in enumerate(sets):
            gs = [dev(synth.numpy_gradient(r_, c_, 8, 0.1, "f32", [86, k, i, step])) for i, (r_, c_) in
                  enumerate(shapes)]
            for (W, G, B), g in zip(refs[k], gs):
                G.copy_(g)
            mm.muon_step([(W, G, B, 1.0) for W, G, B in refs[k]])
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                for (W, G, B), g in zip(bufs[k], gs):
                    G.copy_(g)
            plans[k].step(stream=side)
        side.synchronize()
        for k in range(2):
            for (W, _, B), (Wr, _, Br) in zip(bufs[k], refs[k]):
                assert torch.equal(W, Wr) and torch.equal(B, Br)
    for p in plans:
        p.close()


def test_plan_own_workspace_outlives_a_side_stream_replay(mm):
    """A plan whose workspace the binding allocated (on the current stream)
    is replayed on a side stream and closed without a synchronisation;
    close() returns once the replay has ended (muon_plan_destroy waits for
    it) and only then releases the workspace.  The current stream then
    allocates a buffer of the workspace's size and fills it with a snapshot
    of the workspace (so that, were the block handed out too early, the
    replay would read stale iterates, never a different descriptor table).
    The replay's results equal the eager step's."""
    print("[case] plan workspace, side-stream replay, early close", flush=True)
    shapes = [(768, 3072), (3072, 768), (256, 256)]
    w0 = [(0.02 * np.random.default_rng([87, i]).standard_normal(s)).astype(np.float32) for i, s in enumerate(shapes)]
    gs = [dev(g) for g in _grads(shapes, 0)]
    ref = [(dev(w), g.clone(), torch.zeros(s, device="cuda")) for w, g, s in zip(w0, gs, shapes)]
    mine = [(dev(w), g.clone(), torch.zeros(s, device="cuda")) for w, g, s in zip(w0, gs, shapes)]
    mm.muon_step([(W, G, B, 1.0) for W, G, B in ref])
    plan = mm.muon_plan_create([(W, G, B, 1.0) for W, G, B in mine])
    torch.cuda.synchronize()
    snapshot = plan._own_ws.clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    plan.step(stream=side)
    plan.close()
    del plan
    filler = torch.empty_like(snapshot)
    filler.copy_(snapshot)
    torch.cuda.synchronize()
    for (W, _, B), (Wr, _, Br) in zip(mine, ref):
        assert torch.equal(W, Wr) and torch.equal(B, Br)


def test_plan_replays_on_alternating_streams_are_ordered(mm):
    """Replays of one plan on two streams, alternating, with no
    synchronisation between them: the library orders each replay after the
    previous one, so three replays equal three eager steps on the same
    gradient."""
    print("[case] plan replays alternating streams", flush=True)
    shapes = [(512, 640), (640, 512), (96, 300)]
    w0 = [(0.02 * np.random.default_rng([88, i]).standard_normal(s)).astype(np.float32) for i, s in enumerate(shapes)]
    gs = [dev(g) for g in _grads(shapes, 1)]
    ref = [(dev(w), g.clone(), torch.zeros(s, device="cuda")) for w, g, s in zip(w0, gs, shapes)]
    mine = [(dev(w), g.clone(), torch.zeros(s, device="cuda")) for w, g, s in zip(w0, gs, shapes)]
    for _ in range(3):
        mm.muon_step([(W, G, B, 1.0) for W, G, B in ref])
    plan = mm.muon_plan_create([(W, G, B, 1.0) for W, G, B in mine])
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    plan.step(stream=s1)
    plan.step(stream=s2)
    plan.step(stream=s1)
    plan.close()
    torch.cuda.synchronize()
    for (W, _, B), (Wr, _, Br) in zip(mine, ref):
        assert torch.equal(W, Wr) and torch.equal(B, Br)


def test_plan_destroyed_without_replay(mm):
    """A plan closed without any replay leaves its buffers untouched."""
    shapes = [(256, 256)]
    W = torch.full(shapes[0], 0.5, device="cuda")
    G = torch.ones(shapes[0], device="cuda")
    B = torch.zeros(shapes[0], device="cuda")
    plan = mm.muon_plan_create([(W, G, B, 1.0)])
    plan.close()
    torch.cuda.synchronize()
    assert torch.all(W == 0.5) and torch.all(B == 0)
