"""ctypes binding of libmuon (include/muon.h).  Argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
torch tensors on the current HIP device; torch supplies device memory and
streams, nothing else.  Buffers the binding allocates for a call (workspace,
outputs, the diagnostics array) are allocated on the stream the call runs on.  There is no fallback: if libmuon.so is absent
the first call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading
from typing import List, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuon.so")

MUON_OK = 0
MUON_ERR_INVALID_ARG = -1
MUON_ERR_UNSUPPORTED = -2
MUON_ERR_WORKSPACE = -3
MUON_ERR_ALIAS = -4
MUON_ERR_ALIGN = -5
MUON_ERR_HIP = -6
MUON_F32 = 0
MUON_BF16 = 1
MUON_MAX_NS_STEPS = 64
MUON_MAX_DIM = 65536
MUON_MAX_GRAM = 16384
MUON_COPY_PROBE_VARIANTS = 6
MUON_STATIC_WORKSPACE_BYTES = 64 * 1024 * 1024
STAGES = ("momentum", "norm", "prep", "gram", "poly", "bx", "update", "upload", "bx_update", "diag")
MUON_STAGE_COUNT = len(STAGES)


class muon_matrix_t(ctypes.Structure):
    _fields_ = [
        ("W", ctypes.c_void_p),
        ("G", ctypes.c_void_p),
        ("B", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("scale", ctypes.c_float),
    ]


class muon_hparams_t(ctypes.Structure):
    _fields_ = [
        ("mu", ctypes.c_float),
        ("lr", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("ns_steps", ctypes.c_int32),
        ("nesterov", ctypes.c_int32),
        ("g_dtype", ctypes.c_int32),
        ("weight_decay", ctypes.c_float),
    ]


class muon_diag_t(ctypes.Structure):
    _fields_ = [
        ("momentum_norm", ctypes.c_float),
        ("direction_rms", ctypes.c_float),
        ("update_rms", ctypes.c_float),
        ("weight_rms", ctypes.c_float),
        ("nonfinite", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 3),
    ]


DIAG_FIELDS = ("momentum_norm", "direction_rms", "update_rms", "weight_rms", "nonfinite")


class muon_plan_info_t(ctypes.Structure):
    _fields_ = [
        ("workspace_bytes", ctypes.c_int64),
        ("launches", ctypes.c_int64),
        ("gram_tiles", ctypes.c_int64),
        ("poly_tiles", ctypes.c_int64),
        ("bx_tiles", ctypes.c_int64),
        ("ew_blocks", ctypes.c_int64),
        ("tile", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class muon_matrix_plan_t(ctypes.Structure):
    _fields_ = [
        ("transposed", ctypes.c_int32),
        ("m", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("m_pad", ctypes.c_int32),
        ("n_pad", ctypes.c_int32),
        ("tile", ctypes.c_int32),
        ("bx_tile_rows", ctypes.c_int32),
        ("bx_tile_cols", ctypes.c_int32),
        ("fused_update", ctypes.c_int32),
        ("xcd_edges", ctypes.c_int32),
        ("x_offset", ctypes.c_int64),
    ]


class muon_qk_clip_matrix_t(ctypes.Structure):
    _fields_ = [
        ("W", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("head_dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("max_logit", ctypes.c_void_p),
    ]


class MuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{muon_status_string(status)}: {message}")
        self.status = status


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded libmuon.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m matrix_muon_step_amd.build`; there is no fallback path")
                L = ctypes.CDLL(LIB_PATH)
                P = ctypes.POINTER
                L.muon_workspace_bytes.restype = ctypes.c_size_t
                L.muon_workspace_bytes.argtypes = [P(muon_matrix_t), ctypes.c_int64, P(muon_hparams_t)]
                L.muon_step.restype = ctypes.c_int
                L.muon_step.argtypes = [P(muon_matrix_t), ctypes.c_int64, P(muon_hparams_t),
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
                L.muon_step_static.restype = ctypes.c_int
                L.muon_step_static.argtypes = [P(muon_matrix_t), ctypes.c_int64, P(muon_hparams_t), ctypes.c_void_p]
                L.muon_plan_create.restype = ctypes.c_int
                L.muon_plan_create.argtypes = [P(muon_matrix_t), ctypes.c_int64, P(muon_hparams_t), ctypes.c_void_p,
                                               ctypes.c_size_t, ctypes.c_void_p, P(ctypes.c_void_p)]
                L.muon_plan_step.restype = ctypes.c_int
                L.muon_plan_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
                L.muon_plan_destroy.restype = ctypes.c_int
                L.muon_plan_destroy.argtypes = [ctypes.c_void_p]
                L.muon_step_diag.restype = ctypes.c_int
                L.muon_step_diag.argtypes = [P(muon_matrix_t), ctypes.c_int64, P(muon_hparams_t),
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.c_void_p]
                L.muon_orthogonalize_workspace_bytes.restype = ctypes.c_size_t
                L.muon_orthogonalize_workspace_bytes.argtypes = [
                    P(ctypes.c_int64), P(ctypes.c_int64), ctypes.c_int64, ctypes.c_int32]
                L.muon_orthogonalize.restype = ctypes.c_int
                L.muon_orthogonalize.argtypes = [
                    P(ctypes.c_void_p), P(ctypes.c_void_p), P(ctypes.c_int64), P(ctypes.c_int64),
                    ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                    ctypes.c_size_t, ctypes.c_void_p]
                L.muon_plan_query.restype = ctypes.c_int
                L.muon_plan_query.argtypes = [P(muon_matrix_t), ctypes.c_int64, P(muon_hparams_t),
                                              P(muon_plan_info_t), P(muon_matrix_plan_t)]
                L.muon_profile_enable.restype = ctypes.c_int
                L.muon_profile_enable.argtypes = [ctypes.c_int32]
                L.muon_profile_read.restype = ctypes.c_int
                L.muon_profile_read.argtypes = [P(ctypes.c_double), P(ctypes.c_int64)]
                L.muon_qk_clip.restype = ctypes.c_int
                L.muon_qk_clip.argtypes = [P(muon_qk_clip_matrix_t), ctypes.c_int64, ctypes.c_float,
                                           ctypes.c_void_p]
                L.muon_copy_probe.restype = ctypes.c_int
                L.muon_copy_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                              ctypes.c_void_p]
                L.muon_status_string.restype = ctypes.c_char_p
                L.muon_status_string.argtypes = [ctypes.c_int]
                L.muon_last_error.restype = ctypes.c_char_p
                L.muon_last_error.argtypes = []
                L.muon_abi_version.restype = ctypes.c_int32
                L.muon_abi_version.argtypes = []
                _lib = L
    return _lib


# ---------------------------------------------------------------- small helpers
def muon_abi_version() -> int:
    return int(lib().muon_abi_version())


def muon_status_string(status: int) -> str:
    return lib().muon_status_string(int(status)).decode()


def muon_last_error() -> str:
    return lib().muon_last_error().decode()


def _check(status: int) -> None:
    if status != MUON_OK:
        raise MuonError(status, muon_last_error())


def hparams(mu=0.95, lr=0.02, eps=1e-7, ns_steps=5, nesterov=False, g_dtype=MUON_F32,
            weight_decay=0.0) -> muon_hparams_t:
    return muon_hparams_t(float(mu), float(lr), float(eps), int(ns_steps), int(bool(nesterov)), int(g_dtype),
                          float(weight_decay))


def raw_matrix_array(entries: Sequence[Tuple[int, int, int, int, int, float]]):
    """Builds a muon_matrix_t[] from (W, G, B, rows, cols, scale) integer addresses."""
    arr = (muon_matrix_t * max(1, len(entries)))()
    for i, (w, g, b, r, c, s) in enumerate(entries):
        arr[i] = muon_matrix_t(w, g, b, int(r), int(c), float(s))
    return arr


def _tensor_entries(matrices):
    import torch

    entries = []
    g_dtype = None
    device = None
    for k, mt in enumerate(matrices):
        W, G, B = mt[0], mt[1], mt[2]
        scale = float(mt[3]) if len(mt) > 3 else 1.0
        for name, t in (("W", W), ("G", G), ("B", B)):
            if not t.is_cuda:
                raise ValueError(f"matrix {k}: {name} must be a GPU tensor")
            device = _same_device(device, t, f"matrix {k}: {name}")
            if t.dim() != 2 or not t.is_contiguous():
                raise ValueError(f"matrix {k}: {name} must be a contiguous 2-D tensor")
        if W.dtype != torch.float32 or B.dtype != torch.float32:
            raise ValueError(f"matrix {k}: W and B must be float32")
        if G.dtype == torch.float32:
            gd = MUON_F32
        elif G.dtype == torch.bfloat16:
            gd = MUON_BF16
        else:
            raise ValueError(f"matrix {k}: G must be float32 or bfloat16")
        if g_dtype is None:
            g_dtype = gd
        elif g_dtype != gd:
            raise ValueError("all gradients of one call must share a dtype")
        if W.shape != G.shape or W.shape != B.shape:
            raise ValueError(f"matrix {k}: W, G and B shapes differ")
        entries.append((W.data_ptr(), G.data_ptr(), B.data_ptr(), W.shape[0], W.shape[1], scale))
    return entries, (MUON_F32 if g_dtype is None else g_dtype), device


def _same_device(device, t, what):
    """The device of a call: every tensor of it on one GPU (the library
    launches on the current device, which the call sets to that one)."""
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, other tensors of the call on {device}")
    return t.device


def _torch_stream(stream, device=None):
    """The torch stream object the call runs on: the current stream of
    `device` (default: the current device) for None, a torch stream as given
    (it must belong to `device`), or an external HIP stream handle (int)."""
    import torch

    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream, device=device)
    if device is not None and stream.device != device:
        raise ValueError(f"the stream belongs to {stream.device}, the call's tensors to {device}")
    return stream


@contextlib.contextmanager
def _on(device, stream):
    """Runs a call with `device` current and its stream entered (so that
    allocations made for the call belong to that stream); yields the stream."""
    import torch

    if device is None:
        st = _torch_stream(stream)
        with torch.cuda.stream(st):
            yield st
        return
    with torch.cuda.device(device):
        st = _torch_stream(stream, device)
        with torch.cuda.stream(st):
            yield st


def _alloc_workspace(nbytes: int, device):
    """Workspace on the current stream (callers enter the call's stream first,
    so torch's caching allocator only hands the block to later work that is
    ordered after the call's kernels)."""
    import torch

    if nbytes == 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("torch returned a workspace that is not 256-byte aligned")
    return ws


def _ws_args(workspace, device=None):
    """Pointer and byte size of a workspace tensor; a caller-supplied one must
    be a contiguous GPU tensor on the call's device (the library can only
    check its size and alignment)."""
    if workspace is None:
        return ctypes.c_void_p(0), 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("the workspace must be a contiguous GPU tensor")
    if device is not None and workspace.device != device:
        raise ValueError(f"the workspace is on {workspace.device}, the call's tensors on {device}")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


# ---------------------------------------------------------------- entry points
def muon_workspace_bytes(matrices, mu=0.95, lr=0.02, eps=1e-7, ns_steps=5, nesterov=False,
                         weight_decay=0.0) -> int:
    entries, gd, _ = _tensor_entries(matrices)
    arr = raw_matrix_array(entries)
    hp = hparams(mu, lr, eps, ns_steps, nesterov, gd, weight_decay)
    nbytes = lib().muon_workspace_bytes(arr, len(entries), ctypes.byref(hp))
    if nbytes == 0 and entries:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error())
    return int(nbytes)


def muon_step(matrices, mu=0.95, lr=0.02, ns_steps=5, nesterov=False, eps=1e-7,
              workspace=None, stream=None, weight_decay=0.0) -> None:
    """One Muon step on a list of (W, G, B[, scale]) tensors; W, B updated in place.

    weight_decay is the decoupled decay lambda: W <- W - lr * (lambda * W + scale * O).
    stream: None (torch's current stream), a torch stream, or a HIP stream
    handle (int).  The kernels run on that stream; the caller orders it after
    the work that produced G (and W, B).  A workspace allocated here belongs
    to that stream."""
    entries, gd, device = _tensor_entries(matrices)
    if not entries:
        return
    arr = raw_matrix_array(entries)
    hp = hparams(mu, lr, eps, ns_steps, nesterov, gd, weight_decay)
    need = int(lib().muon_workspace_bytes(arr, len(entries), ctypes.byref(hp)))
    if need == 0:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error())
    with _on(device, stream) as st:
        if workspace is None:
            workspace = _alloc_workspace(need, device)
        ws_ptr, ws_len = _ws_args(workspace, device)
        _check(lib().muon_step(arr, len(entries), ctypes.byref(hp), ws_ptr, ws_len,
                               ctypes.c_void_p(st.cuda_stream)))


def muon_step_static(matrices, mu=0.95, lr=0.02, ns_steps=5, nesterov=False, eps=1e-7, stream=None,
                     weight_decay=0.0) -> None:
    """muon_step with the library's static device workspace: allocates
    nothing (no torch allocation, no hipMalloc).  Raises MuonError
    (MUON_ERR_WORKSPACE) when the call needs more than
    MUON_STATIC_WORKSPACE_BYTES of workspace."""
    entries, gd, device = _tensor_entries(matrices)
    if not entries:
        return
    arr = raw_matrix_array(entries)
    hp = hparams(mu, lr, eps, ns_steps, nesterov, gd, weight_decay)
    with _on(device, stream) as st:
        _check(lib().muon_step_static(arr, len(entries), ctypes.byref(hp), ctypes.c_void_p(st.cuda_stream)))


class MuonPlan:
    """A recorded Muon step on fixed buffers (muon_plan_create).  step()
    replays it; the plan keeps its tensors alive until close()."""

    def __init__(self, handle, keep, device, own_workspace=None):
        self._h = handle
        self._keep = keep
        self._device = device
        self._own_ws = own_workspace  # allocated by muon_plan_create, freed with the plan

    def step(self, stream=None) -> None:
        if not self._h:
            raise RuntimeError("the plan is closed")
        with _on(self._device, stream) as st:
            _check(lib().muon_plan_step(self._h, ctypes.c_void_p(st.cuda_stream)))

    def close(self) -> None:
        """Frees the graph once the last replay has ended (muon_plan_destroy
        waits for it), then releases the tensors the plan kept alive."""
        if self._h:
            h, self._h = self._h, None
            _check(lib().muon_plan_destroy(h))
            self._keep = None
            self._own_ws = None

    def __del__(self):
        try:
            if self._h:
                lib().muon_plan_destroy(self._h)
        except Exception:  # interpreter shutdown
            pass


def muon_plan_create(matrices, mu=0.95, lr=0.02, ns_steps=5, nesterov=False, eps=1e-7, workspace=None,
                     stream=None, weight_decay=0.0) -> MuonPlan:
    """Records one Muon step on these (W, G, B[, scale]) tensors; returns a
    MuonPlan whose step() replays it (write each step's gradient into the
    same G tensors)."""
    entries, gd, device = _tensor_entries(matrices)
    if not entries:
        raise ValueError("a plan needs at least one matrix")
    arr = raw_matrix_array(entries)
    hp = hparams(mu, lr, eps, ns_steps, nesterov, gd, weight_decay)
    need = int(lib().muon_workspace_bytes(arr, len(entries), ctypes.byref(hp)))
    if need == 0:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error())
    own = None
    with _on(device, stream) as st:
        if workspace is None:
            workspace = own = _alloc_workspace(need, device)
        ws_ptr, ws_len = _ws_args(workspace, device)
        h = ctypes.c_void_p()
        _check(lib().muon_plan_create(arr, len(entries), ctypes.byref(hp), ws_ptr, ws_len,
                                      ctypes.c_void_p(st.cuda_stream), ctypes.byref(h)))
    return MuonPlan(h.value, (list(matrices), workspace), device, own)


def muon_step_diag(matrices, mu=0.95, lr=0.02, ns_steps=5, nesterov=False, eps=1e-7,
                   workspace=None, stream=None, weight_decay=0.0, diag=None):
    """muon_step plus per-matrix diagnostics.  Returns the device buffer of
    muon_diag_t records (int32, n x 8; `diag` may supply it); read it with
    diag_records() after the stream is synchronised."""
    import torch

    entries, gd, device = _tensor_entries(matrices)
    n = len(entries)
    if diag is not None:
        if not diag.is_cuda or diag.dtype != torch.int32 or not diag.is_contiguous() or diag.numel() < 8 * n:
            raise ValueError("diag must be a contiguous int32 GPU tensor of at least n x 8 entries")
        device = _same_device(device, diag, "diag")
    with _on(device, stream) as st:
        if diag is None:
            diag = torch.zeros(max(1, n), 8, dtype=torch.int32, device=st.device)
        if not entries:
            return diag
        arr = raw_matrix_array(entries)
        hp = hparams(mu, lr, eps, ns_steps, nesterov, gd, weight_decay)
        need = int(lib().muon_workspace_bytes(arr, n, ctypes.byref(hp)))
        if need == 0:
            raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error())
        if workspace is None:
            workspace = _alloc_workspace(need, device)
        ws_ptr, ws_len = _ws_args(workspace, device)
        _check(lib().muon_step_diag(arr, n, ctypes.byref(hp), ctypes.c_void_p(diag.data_ptr()), ws_ptr, ws_len,
                                    ctypes.c_void_p(st.cuda_stream)))
    return diag


def diag_records(diag, n=None) -> List[dict]:
    """Decodes muon_diag_t records (an int32 n x 8 tensor or array) on the host."""
    import numpy as np

    a = diag.cpu().numpy() if hasattr(diag, "cpu") else np.asarray(diag)
    a = np.ascontiguousarray(a, dtype=np.int32).reshape(-1, 8)
    if n is not None:
        a = a[:n]
    f = a.view(np.float32)
    return [dict(momentum_norm=float(f[i, 0]), direction_rms=float(f[i, 1]), update_rms=float(f[i, 2]),
                 weight_rms=float(f[i, 3]), nonfinite=int(a[i, 4])) for i in range(a.shape[0])]


def muon_orthogonalize_workspace_bytes(shapes: Sequence[Tuple[int, int]], ns_steps=5) -> int:
    n = len(shapes)
    rows = (ctypes.c_int64 * max(1, n))(*[int(s[0]) for s in shapes])
    cols = (ctypes.c_int64 * max(1, n))(*[int(s[1]) for s in shapes])
    nbytes = lib().muon_orthogonalize_workspace_bytes(rows, cols, n, int(ns_steps))
    if nbytes == 0 and n:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error())
    return int(nbytes)


def muon_orthogonalize(Ms, Os=None, ns_steps=5, eps=1e-7, workspace=None, stream=None) -> List:
    """O = NS(M) for a list of float32 matrices; returns the outputs."""
    import torch

    Ms = list(Ms)
    n = len(Ms)
    if n == 0:
        return []
    device = None
    for k, M in enumerate(Ms):
        if M.dtype != torch.float32 or not M.is_cuda:
            raise ValueError(f"matrix {k}: M must be a float32 GPU tensor")
        device = _same_device(device, M, f"matrix {k}: M")
    with _on(device, stream) as st:
        if Os is None:
            Os = [torch.empty_like(M) for M in Ms]
        if len(Os) != n:
            raise ValueError("Os must hold one output per input")
        for k, (M, O) in enumerate(zip(Ms, Os)):
            if O.dtype != torch.float32 or not O.is_cuda:
                raise ValueError(f"matrix {k}: O must be a float32 GPU tensor")
            _same_device(device, O, f"matrix {k}: O")
            if M.shape != O.shape or M.dim() != 2 or not M.is_contiguous() or not O.is_contiguous():
                raise ValueError(f"matrix {k}: M and O must be contiguous 2-D tensors of one shape")
        need = muon_orthogonalize_workspace_bytes([M.shape for M in Ms], ns_steps)
        if workspace is None:
            workspace = _alloc_workspace(need, device)
        mp = (ctypes.c_void_p * n)(*[M.data_ptr() for M in Ms])
        op = (ctypes.c_void_p * n)(*[O.data_ptr() for O in Os])
        rows = (ctypes.c_int64 * n)(*[M.shape[0] for M in Ms])
        cols = (ctypes.c_int64 * n)(*[M.shape[1] for M in Ms])
        ws_ptr, ws_len = _ws_args(workspace, device)
        _check(lib().muon_orthogonalize(mp, op, rows, cols, n, int(ns_steps), float(eps), ws_ptr, ws_len,
                                        ctypes.c_void_p(st.cuda_stream)))
    return Os


def muon_plan_query(shapes: Sequence[Tuple[int, int]], ns_steps=5, g_dtype=MUON_F32):
    """Host-only plan of a step over matrices of these shapes (no GPU needed)."""
    n = len(shapes)
    arr = raw_matrix_array([(0, 0, 0, r, c, 1.0) for r, c in shapes])
    hp = hparams(ns_steps=ns_steps, g_dtype=g_dtype)
    info = muon_plan_info_t()
    per = (muon_matrix_plan_t * max(1, n))()
    _check(lib().muon_plan_query(arr, n, ctypes.byref(hp), ctypes.byref(info), per))
    mats = [dict(transposed=p.transposed, m=p.m, n=p.n, m_pad=p.m_pad, n_pad=p.n_pad,
                 tile=p.tile, bx_tile_rows=p.bx_tile_rows, bx_tile_cols=p.bx_tile_cols, fp32_path=int(p.tile == 0),
                 fused_update=p.fused_update, xcd_edges=p.xcd_edges, x_offset=p.x_offset) for p in list(per)[:n]]
    return {f: getattr(info, f) for f, _ in muon_plan_info_t._fields_ if f != "reserved"}, mats


def muon_profile_enable(on: bool = True) -> None:
    _check(lib().muon_profile_enable(int(bool(on))))


def muon_profile_read():
    """{stage: (milliseconds, launches)} accumulated since the last read."""
    ms = (ctypes.c_double * MUON_STAGE_COUNT)()
    cnt = (ctypes.c_int64 * MUON_STAGE_COUNT)()
    _check(lib().muon_profile_read(ms, cnt))
    return {STAGES[k]: (ms[k], cnt[k]) for k in range(MUON_STAGE_COUNT)}


def muon_copy_probe(src, dst, variant: int = 0, stream=None) -> None:
    """Streaming device copy src -> dst (same byte size) with the library's
    bandwidth yardstick kernel; the HBM ceiling of the bandwidth-bound stages."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not src.is_cuda or not dst.is_cuda:
        raise ValueError("src and dst must be GPU tensors of the same byte size")
    device = _same_device(_same_device(None, src, "src"), dst, "dst")
    with _on(device, stream) as st:
        _check(lib().muon_copy_probe(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                                     int(variant), ctypes.c_void_p(st.cuda_stream)))


def muon_qk_clip(matrices, tau: float, stream=None) -> None:
    """QK-Clip after a step: for each (W, head_dim, max_logit) with W a float32
    (heads * head_dim, cols) projection and max_logit a float32 tensor of
    its heads' max logits, the rows of every head with max_logit > tau are
    scaled by sqrt(tau / max_logit) in place."""
    import torch

    n = len(matrices)
    arr = (muon_qk_clip_matrix_t * max(1, n))()
    device = None
    for k, (W, head_dim, S) in enumerate(matrices):
        if int(head_dim) < 1:
            raise ValueError(f"matrix {k}: head_dim must be >= 1")
        if not W.is_cuda or W.dtype != torch.float32 or W.dim() != 2 or not W.is_contiguous():
            raise ValueError(f"matrix {k}: W must be a contiguous float32 2-D GPU tensor")
        if not S.is_cuda or S.dtype != torch.float32 or not S.is_contiguous():
            raise ValueError(f"matrix {k}: max_logit must be a contiguous float32 GPU tensor")
        device = _same_device(_same_device(device, W, f"matrix {k}: W"), S, f"matrix {k}: max_logit")
        if W.shape[0] % int(head_dim) or S.numel() != W.shape[0] // int(head_dim):
            raise ValueError(f"matrix {k}: rows must be heads * head_dim and max_logit hold one entry per head")
        arr[k] = muon_qk_clip_matrix_t(W.data_ptr(), W.shape[0], W.shape[1], int(head_dim), 0, S.data_ptr())
    with _on(device, stream) as st:
        _check(lib().muon_qk_clip(arr, n, float(tau), ctypes.c_void_p(st.cuda_stream)))
