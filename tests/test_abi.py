"""Host-side checks of libmuon (no GPU): exported symbols, argument
validation (every error is raised before anything is enqueued), and the
execution plan (transpose rule, padding, tile counts, workspace size)."""
import ctypes
import os
import re

import pytest

import matrix_muon_step_amd as mm
from matrix_muon_step_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "muon.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", src)))


def test_header_symbols_exported():
    L = mm.lib()
    names = declared_functions()
    assert "muon_step" in names and "muon_orthogonalize" in names
    for name in names:
        assert hasattr(L, name), name


def test_stage_names_match_header():
    src = open(os.path.join(ROOT, "include", "muon.h")).read()
    enum = {name.lower(): int(v) for name, v in re.findall(r"MUON_STAGE_([A-Z_]+)\s*=\s*(\d+)", src)}
    count = enum.pop("count")
    assert count == len(bd.STAGES) == bd.MUON_STAGE_COUNT
    assert all(bd.STAGES[v] == name for name, v in enum.items())


def test_abi_version_and_strings():
    assert mm.muon_abi_version() == 7
    assert mm.muon_status_string(0) == "MUON_OK"
    assert mm.muon_status_string(-4) == "MUON_ERR_ALIAS"


BASE = 1 << 32  # fake, 256-byte aligned device addresses; never dereferenced


def step(entries, hp=None, ws=BASE * 64, ws_bytes=1 << 40):
    arr = bd.raw_matrix_array(entries)
    hp = hp or bd.hparams()
    return mm.lib().muon_step(arr, len(entries), ctypes.byref(hp), ctypes.c_void_p(ws), ws_bytes, None)


def good(i=0, r=64, c=96):
    return (BASE * (4 * i + 1), BASE * (4 * i + 2), BASE * (4 * i + 3), r, c, 1.0)


def test_n_zero_is_noop():
    hp = bd.hparams()
    assert mm.lib().muon_step(None, 0, ctypes.byref(hp), None, 0, None) == mm.MUON_OK


@pytest.mark.parametrize("mutate,status", [
    (lambda e: (0,) + e[1:], mm.MUON_ERR_INVALID_ARG),                 # W NULL
    (lambda e: e[:1] + (0,) + e[2:], mm.MUON_ERR_INVALID_ARG),         # G NULL
    (lambda e: e[:2] + (0,) + e[3:], mm.MUON_ERR_INVALID_ARG),         # B NULL
    (lambda e: e[:3] + (0,) + e[4:], mm.MUON_ERR_INVALID_ARG),         # rows 0
    (lambda e: e[:4] + (-3,) + e[5:], mm.MUON_ERR_INVALID_ARG),        # cols < 0
    (lambda e: (e[0] + 4,) + e[1:], mm.MUON_ERR_ALIGN),                # W misaligned
    (lambda e: e[:2] + (e[2] + 8,) + e[3:], mm.MUON_ERR_ALIGN),        # B misaligned
    (lambda e: e[:5] + (float("nan"),), mm.MUON_ERR_INVALID_ARG),      # scale NaN
    (lambda e: e[:3] + (70000,) + e[4:], mm.MUON_ERR_UNSUPPORTED),     # rows > MAX_DIM
    (lambda e: e[:3] + (20000, 20000, 1.0), mm.MUON_ERR_UNSUPPORTED),  # Gram side > MAX_GRAM
    (lambda e: e[:2] + (e[0] + 256,) + e[3:], mm.MUON_ERR_ALIAS),      # B inside W
    (lambda e: (e[1],) + e[1:], mm.MUON_ERR_ALIAS),                    # W == G
])
def test_matrix_argument_errors(mutate, status):
    e = mutate(good())
    assert step([good(1), e]) == status
    assert mm.muon_last_error() != ""


def test_cross_matrix_alias():
    a = good(0)
    b = (a[0] + 64 * 4 * 10,) + good(1)[1:]  # W of matrix 1 inside W of matrix 0
    assert step([a, b]) == mm.MUON_ERR_ALIAS


def test_shared_gradient_is_allowed_for_validation():
    # Two matrices reading one G (read-only) is not an alias; the call then
    # fails only because there is no GPU / the address is fake, so check the
    # validation layer via the workspace query instead.
    a = good(0)
    b = good(1)[:1] + (a[1],) + good(1)[2:]
    arr = bd.raw_matrix_array([a, b])
    hp = bd.hparams()
    assert mm.lib().muon_workspace_bytes(arr, 2, ctypes.byref(hp)) > 0


def test_workspace_overlap_is_alias():
    a = good(0)
    assert step([a], ws=a[0]) == mm.MUON_ERR_ALIAS


@pytest.mark.parametrize("kw,status", [
    (dict(ns_steps=-1), mm.MUON_ERR_INVALID_ARG),
    (dict(ns_steps=65), mm.MUON_ERR_INVALID_ARG),
    (dict(eps=-1.0), mm.MUON_ERR_INVALID_ARG),
    (dict(mu=float("inf")), mm.MUON_ERR_INVALID_ARG),
    (dict(lr=float("nan")), mm.MUON_ERR_INVALID_ARG),
    (dict(g_dtype=7), mm.MUON_ERR_INVALID_ARG),
    (dict(weight_decay=float("nan")), mm.MUON_ERR_INVALID_ARG),
    (dict(weight_decay=float("inf")), mm.MUON_ERR_INVALID_ARG),
])
def test_hparam_errors(kw, status):
    assert step([good()], hp=bd.hparams(**kw)) == status


def test_nesterov_must_be_boolean():
    hp = bd.hparams()
    hp.nesterov = 2
    assert step([good()], hp=hp) == mm.MUON_ERR_INVALID_ARG


def test_workspace_errors():
    e = [good()]
    arr = bd.raw_matrix_array(e)
    hp = bd.hparams()
    need = mm.lib().muon_workspace_bytes(arr, 1, ctypes.byref(hp))
    assert need > 0
    assert step(e, ws=0) == mm.MUON_ERR_WORKSPACE
    assert step(e, ws=BASE * 64 + 128) == mm.MUON_ERR_WORKSPACE
    assert step(e, ws_bytes=need - 1) == mm.MUON_ERR_WORKSPACE


def test_null_descriptor_arrays():
    hp = bd.hparams()
    assert mm.lib().muon_step(None, 2, ctypes.byref(hp), None, 0, None) == mm.MUON_ERR_INVALID_ARG
    arr = bd.raw_matrix_array([good()])
    assert mm.lib().muon_step(arr, 1, None, None, 0, None) == mm.MUON_ERR_INVALID_ARG
    assert mm.lib().muon_step(arr, -1, ctypes.byref(hp), None, 0, None) == mm.MUON_ERR_INVALID_ARG


def test_orthogonalize_errors():
    L = mm.lib()
    rows = (ctypes.c_int64 * 1)(8)
    cols = (ctypes.c_int64 * 1)(8)
    M = (ctypes.c_void_p * 1)(BASE)
    O = (ctypes.c_void_p * 1)(BASE + 4)
    assert L.muon_orthogonalize(M, O, rows, cols, 1, 5, 1e-7, ctypes.c_void_p(BASE * 64), 1 << 40, None) == mm.MUON_ERR_ALIGN
    O2 = (ctypes.c_void_p * 1)(BASE)
    assert L.muon_orthogonalize(M, O2, rows, cols, 1, 5, 1e-7, ctypes.c_void_p(BASE * 64), 1 << 40, None) == mm.MUON_ERR_ALIAS
    assert L.muon_orthogonalize(M, O2, rows, cols, 1, 5, -1.0, None, 0, None) == mm.MUON_ERR_INVALID_ARG
    assert L.muon_orthogonalize(None, None, rows, cols, 0, 5, 1e-7, None, 0, None) == mm.MUON_OK


# ------------------------------------------------------------------ plan
def test_plan_transpose_rule_and_padding():
    shapes = [(1600, 1600), (1600, 6400), (6400, 1600), (33, 17), (17, 33), (1, 1), (2048, 7168),
              (768, 3072), (100, 300)]
    info, mats = mm.muon_plan_query(shapes)
    assert [m["transposed"] for m in mats] == [0, 0, 1, 1, 0, 0, 0, 0, 0]
    for m, (r, c) in zip(mats, shapes):
        assert m["m"] == min(r, c) and m["n"] == max(r, c)
        assert m["x_offset"] % 256 == 0
        if m["m"] <= 64:
            # float32 small-Gram path: 64 x (n rounded up to 256)
            assert m["tile"] == 0 and m["fp32_path"] == 1 and m["m_pad"] == 64
            assert m["n_pad"] % 256 == 0 and m["n"] <= m["n_pad"] < m["n"] + 256
        else:
            t, tr, tc = m["tile"], m["bx_tile_rows"], m["bx_tile_cols"]
            assert t in (128, 160, 256) and tc in (128, 160, 256) and m["fp32_path"] == 0
            assert tr in (128, 160, 256, 320)
            assert m["m_pad"] % t == 0 and m["m_pad"] % tr == 0 and m["m"] <= m["m_pad"] < m["m"] + max(t, tr)
            assert m["n_pad"] % tc == 0 and m["n"] <= m["n_pad"] < m["n"] + tc
    # Tile choice: exact fits are preferred (1600 = 10 x 160 = 5 x 320); the
    # 256-tile matrices of this call (2048 x 7168, 768 x 3072: 260 BX tiles)
    # run on 128-tiles, as every call with fewer than 512 such tiles does.
    assert [m["tile"] for m in mats] == [160, 160, 160, 0, 0, 0, 128, 128, 128]
    assert [m["bx_tile_rows"] for m in mats] == [320, 320, 320, 0, 0, 0, 128, 128, 128]


def test_plan_small_call_uses_128_tiles():
    """A call whose 256-tile BX launch would hold fewer than 512 tiles runs
    those matrices on 128-tiles (same arithmetic); from 512 tiles on, 256."""
    one = [(2048, 7168)]                      # 8 x 28 = 224 BX tiles of 256
    _, mats = mm.muon_plan_query(one)
    assert mats[0]["tile"] == 128 and mats[0]["bx_tile_rows"] == 128 and mats[0]["m_pad"] == 2048
    _, mats = mm.muon_plan_query(one * 3)     # 672 tiles
    assert all(m["tile"] == 256 and m["bx_tile_rows"] == 256 for m in mats)
    # exactly at the threshold: 2 x (8 x 28) + 64 x ... -> 512 tiles keep 256
    _, mats = mm.muon_plan_query(one * 2 + [(256, 256)] * 64)   # 448 + 64 = 512
    assert all(m["tile"] == 256 for m in mats)
    _, mats = mm.muon_plan_query(one * 2 + [(256, 256)] * 63)   # 511
    assert all(m["tile"] == 128 for m in mats)
    # the 1600-class (160/320 tiles) and float32-path matrices are unaffected
    _, mats = mm.muon_plan_query([(1600, 1600), (40, 90)] + one)
    assert [m["tile"] for m in mats] == [160, 0, 128]


def test_plan_small_path_threshold():
    info, mats = mm.muon_plan_query([(64, 1000), (1000, 64), (65, 1000), (1000, 65)])
    assert [m["fp32_path"] for m in mats] == [1, 1, 0, 0]
    # Small matrices add no matrix-core tiles; mixing both paths adds launches.
    assert info["launches"] == 4 + 2 * 3 * 5
    info_big, big = mm.muon_plan_query([(65, 1000), (1000, 65)])
    assert info_big["gram_tiles"] == info["gram_tiles"] and info_big["bx_tiles"] == info["bx_tiles"]
    assert info_big["launches"] == 3 + _update_launch(big) + 3 * 5


def test_plan_tile_counts_and_workspace():
    shapes = [(1600, 1600)] * 4 + [(1600, 6400), (6400, 1600)]
    info, mats = mm.muon_plan_query(shapes, ns_steps=5)
    sym = sum((m["m_pad"] // m["tile"]) * (m["m_pad"] // m["tile"] + 1) // 2 for m in mats)
    bx = sum((m["m_pad"] // m["bx_tile_rows"]) * (m["n_pad"] // m["bx_tile_cols"]) for m in mats)
    assert info["gram_tiles"] == sym == info["poly_tiles"]
    assert info["bx_tiles"] == bx
    assert info["launches"] == 3 + _update_launch(mats) + 3 * 5
    # four bf16 copies of the iterate (two hi/lo pairs of X^T, ping-pong) + A + P
    floor = sum(4 * 2 * m["m_pad"] * m["n_pad"] + 2 * 2 * m["m_pad"] ** 2 for m in mats)
    assert floor <= info["workspace_bytes"] <= floor + (1 << 20)
    info0, _ = mm.muon_plan_query(shapes, ns_steps=0)
    assert info0["workspace_bytes"] < info["workspace_bytes"]
    assert info0["launches"] == 4


def test_plan_momentum_tiles_follow_orientation():
    """The momentum pass takes tiles of 64 rows x 128 columns of M in M's own
    orientation: 64 x 128 of the padded short-side-major X when M is stored
    as is, 128 x 64 when it is transposed (rows > cols)."""
    def cdiv(a, b):
        return -(-a // b)
    shapes = [(1600, 6400), (6400, 1600), (1600, 1600), (65, 300), (300, 65), (63, 4097), (4097, 63)]
    total = 0
    for s in shapes:
        info, (m,) = mm.muon_plan_query([s])
        tr = s[0] > s[1]
        ti, tj = (128, 64) if tr else (64, 128)
        expect = cdiv(m["m_pad"], ti) * cdiv(m["n_pad"], tj)
        assert info["ew_blocks"] == expect, (s, info["ew_blocks"], expect)
        total += expect
    assert mm.muon_plan_query(shapes)[0]["ew_blocks"] == total


def test_plan_mixed_tiles_launch_groups():
    # 1600: 160-tile symmetric products and 320-row BX tiles; 2048 (a small
    # call: 64 BX tiles of 256) on the 32x32 128-tiles; 100 x 300 on the
    # 16x16 128-tiles: three configurations per stage.
    info, mats = mm.muon_plan_query([(1600, 1600), (2048, 2048), (100, 300)], ns_steps=5)
    assert [m["tile"] for m in mats] == [160, 128, 128]
    assert [m["fused_update"] for m in mats] == [1, 1, 0]
    assert info["launches"] == 3 + _update_launch(mats) + 3 * 3 * 5


def _update_launch(mats):
    """1 when some matrix still needs the separate update pass."""
    return int(any(m["fused_update"] == 0 for m in mats))


def test_plan_fused_update_flags():
    """The wide-tile BX kernels (32x32x16 products: 256-, 128-, 320x256- and
    160x256-tiles) apply the update in their last launch; the float32 path,
    the 16x16 tiles and ns_steps = 0 keep the separate update pass."""
    shapes = [(2048, 7168), (7168, 2048), (1600, 1600), (100, 300), (33, 17)]
    info, mats = mm.muon_plan_query(shapes, ns_steps=5)
    assert [m["fused_update"] for m in mats] == [1, 1, 1, 0, 0]
    big, _ = mm.muon_plan_query(shapes[:2] * 2, ns_steps=5)   # 896 BX tiles: 256-tiles
    assert big["tile"] == 256
    info_w, _ = mm.muon_plan_query(shapes[:2], ns_steps=5)
    assert info_w["launches"] == 3 + 3 * 5
    _, mats0 = mm.muon_plan_query(shapes, ns_steps=0)
    assert all(m["fused_update"] == 0 for m in mats0)


def test_plan_limits():
    with pytest.raises(mm.MuonError):
        mm.muon_plan_query([(0, 5)])
    info, _ = mm.muon_plan_query([(16384, 65536)])
    assert info["workspace_bytes"] > 0
    with pytest.raises(mm.MuonError):
        mm.muon_plan_query([(16385, 16385)])


def test_copy_probe_errors():
    L = mm.lib()
    a, b = BASE * 2, BASE * 3
    assert L.muon_copy_probe(None, b, 64, 0, None) == mm.MUON_ERR_INVALID_ARG
    assert L.muon_copy_probe(a + 8, b, 64, 0, None) == mm.MUON_ERR_ALIGN
    assert L.muon_copy_probe(a, b, 60, 0, None) == mm.MUON_ERR_ALIGN
    assert L.muon_copy_probe(a, a + 32, 64, 0, None) == mm.MUON_ERR_ALIAS
    assert L.muon_copy_probe(a, b, 64, -1, None) == mm.MUON_ERR_INVALID_ARG
    assert L.muon_copy_probe(a, b, 64, bd.MUON_COPY_PROBE_VARIANTS, None) == mm.MUON_ERR_INVALID_ARG
    assert L.muon_copy_probe(a, b, 0, 0, None) == mm.MUON_OK


def test_plan_xcd_edges_uniform_layers():
    """48 identical layers of 6 matrices: each of the 8 XCDs takes 6 whole
    layers of every grouped launch, so the XCD shares start exactly at
    matrices 36, 72, ..., 252, in the Gram, polynomial and BX launches."""
    import synth
    w = synth.WORKLOADS["gpt2_xl_1p5b"]
    _, plans = mm.muon_plan_query([(s.rows, s.cols) for s in w.matrices])
    edges = {i: p["xcd_edges"] for i, p in enumerate(plans) if p["xcd_edges"]}
    assert edges == {36 * k: 7 for k in range(1, 8)}


def test_plan_xcd_edges_single_matrix():
    """One matrix with many tiles: every XCD share starts inside it."""
    _, plans = mm.muon_plan_query([(2048, 7168)])
    assert plans[0]["xcd_edges"] == 7
    _, plans = mm.muon_plan_query([(40, 70)])   # float32 path: no matrix-core launch
    assert plans[0]["xcd_edges"] == 0


def test_step_static_rejects_before_any_gpu_call():
    """muon_step_static validates and sizes the call on the host: arguments
    errors and a workspace beyond the static array come back without a GPU
    (this container has none) and without touching the device."""
    L = mm.lib()
    hp = bd.hparams()
    assert L.muon_step_static(None, 0, ctypes.byref(hp), None) == mm.MUON_OK
    arr = bd.raw_matrix_array([good(0, 4096, 4096)])
    assert L.muon_step_static(arr, 1, ctypes.byref(hp), None) == mm.MUON_ERR_WORKSPACE
    msg = mm.muon_last_error()
    assert "static workspace holds" in msg and str(bd.MUON_STATIC_WORKSPACE_BYTES) in msg
    arr = bd.raw_matrix_array([(0, BASE * 2, BASE * 3, 64, 64, 1.0)])
    assert L.muon_step_static(arr, 1, ctypes.byref(hp), None) == mm.MUON_ERR_INVALID_ARG
    bad_hp = bd.hparams(ns_steps=-1)
    arr = bd.raw_matrix_array([good(0)])
    assert L.muon_step_static(arr, 1, ctypes.byref(bad_hp), None) == mm.MUON_ERR_INVALID_ARG


def test_static_workspace_size_matches_header():
    src = open(os.path.join(ROOT, "include", "muon.h")).read()
    m = re.search(r"#define MUON_STATIC_WORKSPACE_BYTES \((\d+)u \* 1024u \* 1024u\)", src)
    assert m and int(m.group(1)) * 2**20 == bd.MUON_STATIC_WORKSPACE_BYTES


def _clip_arr(entries):
    arr = (bd.muon_qk_clip_matrix_t * max(1, len(entries)))()
    for k, (w, r, c, hd, s) in enumerate(entries):
        arr[k] = bd.muon_qk_clip_matrix_t(w, r, c, hd, 0, s)
    return arr


@pytest.mark.parametrize("entry,tau,status", [
    ((BASE, 64, 32, 16, BASE * 2), 0.0, "MUON_ERR_INVALID_ARG"),          # tau must be > 0
    ((BASE, 64, 32, 16, BASE * 2), float("inf"), "MUON_ERR_INVALID_ARG"),
    ((BASE, 64, 32, 16, BASE * 2), float("nan"), "MUON_ERR_INVALID_ARG"),
    ((0, 64, 32, 16, BASE * 2), 1.0, "MUON_ERR_INVALID_ARG"),             # NULL W
    ((BASE, 64, 32, 16, 0), 1.0, "MUON_ERR_INVALID_ARG"),                 # NULL max_logit
    ((BASE, 64, 32, 0, BASE * 2), 1.0, "MUON_ERR_INVALID_ARG"),           # head_dim 0
    ((BASE, 64, 32, 24, BASE * 2), 1.0, "MUON_ERR_INVALID_ARG"),          # rows % head_dim
    ((BASE, 0, 32, 16, BASE * 2), 1.0, "MUON_ERR_INVALID_ARG"),
    ((BASE + 4, 64, 32, 16, BASE * 2), 1.0, "MUON_ERR_ALIGN"),
    ((BASE, 64, 32, 16, BASE * 2 + 2), 1.0, "MUON_ERR_ALIGN"),
    ((BASE, 64, 70000, 16, BASE * 2), 1.0, "MUON_ERR_UNSUPPORTED"),
    ((BASE, 64, 32, 16, BASE + 64), 1.0, "MUON_ERR_ALIAS"),               # max_logit inside W
])
def test_qk_clip_argument_errors(entry, tau, status):
    L = mm.lib()
    assert mm.muon_status_string(L.muon_qk_clip(_clip_arr([entry]), 1, tau, None)) == status


def test_qk_clip_cross_matrix_alias_and_shared_logits():
    L = mm.lib()
    # two matrices whose W overlap: refused
    arr = _clip_arr([(BASE, 64, 32, 16, BASE * 3), (BASE + 1024, 64, 32, 16, BASE * 3)])
    assert L.muon_qk_clip(arr, 2, 1.0, None) == mm.MUON_ERR_ALIAS
    # n == 0 is a no-op; a NULL list with n > 0 is refused
    assert L.muon_qk_clip(None, 0, 1.0, None) == mm.MUON_OK
    assert L.muon_qk_clip(None, 1, 1.0, None) == mm.MUON_ERR_INVALID_ARG


def test_plan_create_rejects_before_any_gpu_call():
    """muon_plan_create validates like muon_step (no GPU in this container:
    every error below comes back before the first HIP call)."""
    L = mm.lib()
    hp = bd.hparams()
    h = ctypes.c_void_p()
    arr = bd.raw_matrix_array([good(0)])
    assert L.muon_plan_create(arr, 1, ctypes.byref(hp), ctypes.c_void_p(BASE * 64), 1 << 40, None, None) \
        == mm.MUON_ERR_INVALID_ARG                                       # out is NULL
    assert L.muon_plan_create(arr, 0, ctypes.byref(hp), ctypes.c_void_p(BASE * 64), 1 << 40, None,
                              ctypes.byref(h)) == mm.MUON_ERR_INVALID_ARG  # no matrix
    assert L.muon_plan_create(arr, 1, ctypes.byref(hp), ctypes.c_void_p(BASE * 64), 16, None,
                              ctypes.byref(h)) == mm.MUON_ERR_WORKSPACE
    assert L.muon_plan_create(arr, 1, ctypes.byref(hp), ctypes.c_void_p(BASE * 64 + 8), 1 << 40, None,
                              ctypes.byref(h)) == mm.MUON_ERR_WORKSPACE
    bad = bd.raw_matrix_array([good(0), (BASE * 1 + 64, BASE * 6, BASE * 7, 64, 96, 1.0)])
    assert L.muon_plan_create(bad, 2, ctypes.byref(hp), ctypes.c_void_p(BASE * 64), 1 << 40, None,
                              ctypes.byref(h)) == mm.MUON_ERR_ALIAS
    assert h.value is None
    assert L.muon_plan_destroy(None) == mm.MUON_OK
    assert L.muon_plan_step(None, None) == mm.MUON_ERR_INVALID_ARG


def test_binding_rejects_tensors_on_two_devices():
    """Every tensor of a call must sit on one device (the binding makes it
    the current device for the call); a second device is refused on the
    host before anything runs."""
    import torch

    a = torch.empty(2, 2)
    b = torch.empty(2, 2, device="meta")
    assert bd._same_device(None, a, "W") == a.device
    assert bd._same_device(a.device, a, "G") == a.device
    with pytest.raises(ValueError, match="meta"):
        bd._same_device(a.device, b, "B")


def test_binding_rejects_host_workspace():
    """A caller-supplied workspace must be a contiguous GPU tensor on the
    call's device: a host tensor would reach the kernels as a host address.
    Refused on the host before anything runs."""
    import torch

    with pytest.raises(ValueError, match="GPU tensor"):
        bd._ws_args(torch.empty(1024, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU tensor"):
        bd._ws_args(torch.empty(1024, dtype=torch.uint8, device="meta"))
    assert bd._ws_args(None)[1] == 0


def test_binding_rejects_zero_head_dim():
    import torch

    W = torch.empty(4, 8)
    with pytest.raises(ValueError, match="head_dim"):
        bd.muon_qk_clip([(W, 0, torch.empty(1))], 1.0)
