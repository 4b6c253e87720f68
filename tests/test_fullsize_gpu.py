"""The full-size grouped launches that carry the benchmark figures.

For the 1.5B-shaped set (288 matrices) and the MoE share (136 matrices):
  * every matrix's W and B after one grouped call equal, bit for bit, those
    of one call per matrix on the same inputs (the tile configuration of a
    matrix depends on its shape alone, and nothing of one matrix's
    arithmetic depends on where its tiles run);
  * the first and last matrix, and every matrix at which one of the 8 XCDs
    starts its share of a grouped matrix-core launch (muon_plan_query's
    xcd_edges), against the float64 oracle: B to the float32 bar, the
    applied step to the Newton-Schulz bar.
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


def _full_size(mm, name):
    w = synth.WORKLOADS[name]
    shapes = [(s.rows, s.cols) for s in w.matrices]
    g_dtype = mm.MUON_BF16 if w.g_dtype == "bf16" else mm.MUON_F32
    _, plans = mm.muon_plan_query(shapes, ns_steps=5, g_dtype=g_dtype)
    check = sorted({0, len(shapes) - 1} | {i for i, p in enumerate(plans) if p["xcd_edges"]})
    print(f"[case] {name}: {len(shapes)} matrices grouped vs one by one; oracle on {check}", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234 + w.wid)
    grouped, single, keep = [], [], {}
    for i in range(len(shapes)):
        t = synth.torch_matrix(w, i, 0, "cuda", generator=gen)
        if i in check:
            keep[i] = (t["W0"].cpu().numpy().copy(), t["G"].float().cpu().numpy().astype(np.float64))
        grouped.append((t["W0"], t["G"], t["B0"], w.scale))
        single.append((t["W0"].clone(), t["G"], torch.zeros_like(t["B0"]), w.scale))
    mm.muon_step(grouped, mu=w.mu, lr=w.lr, ns_steps=5)
    torch.cuda.synchronize()
    ws_bytes = max(mm.muon_workspace_bytes([mt], mu=w.mu, lr=w.lr, ns_steps=5) for mt in single[:1] + single[-1:]
                   + [single[i] for i in check])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    for mt in single:
        mm.muon_step([mt], mu=w.mu, lr=w.lr, ns_steps=5, workspace=ws)
    torch.cuda.synchronize()
    bad = [i for i in range(len(shapes))
           if not (torch.equal(grouped[i][0], single[i][0]) and torch.equal(grouped[i][2], single[i][2]))]
    print(f"  grouped vs one by one: {len(shapes) - len(bad)} of {len(shapes)} matrices bit-identical", flush=True)
    assert not bad, f"matrices differing between the grouped and the one-by-one calls: {bad[:10]}"
    del single, ws
    for i in check:
        W0, g64 = keep[i]
        Wr, Br, _ = orc.muon_step(W0, g64, np.zeros_like(g64), w.mu, w.lr, w.scale, 5)
        Wg = grouped[i][0].cpu().numpy().astype(np.float64)
        Bg = grouped[i][2].cpu().numpy()
        b_err = relfro(Bg, Br)
        err = relfro(Wg - W0, Wr - W0)
        print(f"  matrix {i} {shapes[i][0]}x{shapes[i][1]} (xcd_edges {plans[i]['xcd_edges']}): "
              f"direction relFro {err:.3e}, momentum relFro {b_err:.3e}", flush=True)
        assert b_err <= FP32_TOL
        assert err <= NS_TOL
    del grouped
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_gpt2_xl_full_size(mm):
    _full_size(mm, "gpt2_xl_1p5b")


@pytest.mark.timeout(900)
def test_moe_share_full_size(mm):
    _full_size(mm, "moe_share")
