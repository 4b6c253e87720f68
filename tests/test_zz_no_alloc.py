"""muon_step_static (the entry point that allocates nothing) against
muon_step, through the C ABI: identical bits on two calls in a row, the
second with a smaller input, and the size limit enforced."""
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


def _inputs(shapes, seed):
    out = []
    for i, (r, c) in enumerate(shapes):
        g = synth.numpy_gradient(r, c, 8, 0.1, "f32", [80, seed, i, 0])
        w0 = (0.02 * np.random.default_rng([80, seed, i, 1]).standard_normal((r, c))).astype(np.float32)
        b0 = (0.01 * np.random.default_rng([80, seed, i, 2]).standard_normal((r, c))).astype(np.float32)
        out.append((w0, g, b0))
    return out


def _check_against_step(mm, shapes, seed, **kw):
    host = _inputs(shapes, seed)
    ref = [(dev(w), dev(g), dev(b), 1.0 + 0.25 * i) for i, (w, g, b) in enumerate(host)]
    got = [(dev(w), dev(g), dev(b), 1.0 + 0.25 * i) for i, (w, g, b) in enumerate(host)]
    need = mm.muon_workspace_bytes(ref, **kw)
    assert need <= mm.MUON_STATIC_WORKSPACE_BYTES
    mm.muon_step(ref, **kw)
    mm.muon_step_static(got, **kw)
    torch.cuda.synchronize()
    for (Wr, _, Br, _), (Wg, _, Bg, _), shp in zip(ref, got, shapes):
        assert torch.equal(Wr, Wg), shp
        assert torch.equal(Br, Bg), shp
    return need


def test_static_step_equals_step_twice_then_smaller(mm):
    print("[case] muon_step_static vs muon_step: two calls, the second smaller", flush=True)
    big = [(768, 3072), (3072, 768), (256, 256), (100, 300), (40, 1000), (1000, 130)]
    small = [(256, 256), (17, 33)]
    n1 = _check_against_step(mm, big, 1)
    n2 = _check_against_step(mm, small, 2, weight_decay=0.1, nesterov=True)
    assert n2 < n1
    # and once more with the first input's shapes (stale contents of the array)
    _check_against_step(mm, big, 3, ns_steps=3)


def test_static_step_rejects_oversize(mm):
    print("[case] muon_step_static size limit", flush=True)
    r, c = 2048, 4096
    mats = [(torch.zeros(r, c, device="cuda"), torch.ones(r, c, device="cuda"), torch.zeros(r, c, device="cuda"), 1.0)]
    assert mm.muon_workspace_bytes(mats) > mm.MUON_STATIC_WORKSPACE_BYTES
    with pytest.raises(mm.MuonError) as ei:
        mm.muon_step_static(mats)
    assert ei.value.status == mm.MUON_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(mats[0][0]).item() == 0 and torch.count_nonzero(mats[0][2]).item() == 0
