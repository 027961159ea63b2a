"""MI355X-native selective state-space scan.

The compute path is the HIP library ``libssm_scan.so`` (C ABI, declared in
``include/ssm_scan.h``). The Python functions here only marshal torch device
tensors into that ABI; the library is loaded on first use and a missing or
unloadable library raises at once.
"""

from .binding import (  # noqa: F401
    ssm_abi_version,
    ssm_causal_conv1d_fwd,
    ssm_causal_conv1d_update,
    ssm_scan_bwd_workspace_bytes,
    ssm_scan_chunks,
    ssm_scan_workspace_bytes,
    ssm_selective_scan_bwd,
    ssm_selective_scan_fwd,
    ssm_selective_state_update,
    ssm_ssd_fwd,
    SSMError,
)
