"""Paged absorbed-MLA attention (PagedAttention, LATENT cache layout) for AMD MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of include/pa_latent.h
(libpa_latent.so, built by `python -m paged_absorbed_mla_amd.build`). This package
holds the ctypes binding with the same entry-point names, torch-based device
plumbing, and the seeded synthetic workload generator.
"""
from ._lib import (  # noqa: F401
    PA_BF16, PA_F16, PA_OK, PA_ERR_CAPTURE_NOT_WARMED, PA_ERR_DEVICE, PA_ERR_INVALID_ARGUMENT,
    PA_ERR_NOT_IMPLEMENTED,
    PA_ERR_WORKSPACE_TOO_SMALL, PaError, load, make_attrs, make_dims, pa_last_error,
    pa_latent_abi_version, pa_latent_attention, pa_latent_attention_noalloc, pa_latent_attention_splits,
    pa_latent_capture_ready, pa_latent_forward, pa_latent_profile_next,
    pa_latent_workspace_size,
    pa_latent_write, pa_separate_attention, pa_separate_forward, pa_separate_workspace_size, pa_separate_write,
)
