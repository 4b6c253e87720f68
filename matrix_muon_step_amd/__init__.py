"""MI355X-native Muon optimizer step: hand-written gfx950 HIP kernels behind
the C ABI of include/muon.h, with a thin ctypes binding of the same names."""
from .binding import (  # noqa: F401
    MUON_OK, MUON_ERR_INVALID_ARG, MUON_ERR_UNSUPPORTED, MUON_ERR_WORKSPACE, MUON_ERR_ALIAS,
    MUON_ERR_ALIGN, MUON_ERR_HIP, MUON_F32, MUON_BF16, MUON_COPY_PROBE_VARIANTS, MuonError, STAGES,
    muon_abi_version, muon_status_string, muon_last_error, muon_workspace_bytes, muon_step,
    muon_step_static, MUON_STATIC_WORKSPACE_BYTES, muon_plan_create, MuonPlan,
    muon_step_diag, diag_records, DIAG_FIELDS,
    muon_orthogonalize_workspace_bytes, muon_orthogonalize, muon_plan_query,
    muon_profile_enable, muon_profile_read, muon_copy_probe, muon_qk_clip, lib, LIB_PATH,
)
