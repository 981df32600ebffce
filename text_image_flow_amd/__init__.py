"""MI355X-native Lens MM-DiT denoiser: hand-written HIP kernels for gfx950
behind a C ABI (include/lens.h), with a thin ctypes binding under the same
names.  ``text_image_flow_amd.device`` holds the PyTorch-side plumbing
(device memory, streams, weight upload, the sampler loop)."""
from ._lib import (  # noqa: F401
    EXPORTS, LENS_BF16, LENS_F32, LENS_MX_ROWS, LENS_MX_SLABS, LENS_OK, LensBlockW, LensConfig, LensDitW, LensError, LensLinear, LensStreamW,
    check, default_config, last_error, lens_block_forward, lens_block_workspace_bytes, lens_dit_forward,
    lens_dit_workspace_bytes, lens_flow_step, lens_flow_step_rescaled, lens_quantize_mxfp8, lens_timer_start,
    lens_timer_stop, lens_time_grid, lens_mu_for_tokens, lib,
    status_string, version,
)
