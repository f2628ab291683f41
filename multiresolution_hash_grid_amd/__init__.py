"""MI355X-native multiresolution hash-grid encoder.

The encoder runs in ``libhashgrid.so`` (HIP kernels for gfx950 behind the C
ABI of ``include/hashgrid.h``); ``hashgrid`` is its Python binding and
``inputs`` the seeded synthetic workload generator.
"""
from .hashgrid import (  # noqa: F401
    HashGridAdam,
    HashGridConfig,
    HashGridEncoder,
    HashGridError,
    HashGridFunction,
    HashGridMLP,
    HashGridMLPFunction,
    abi_version,
    backward_workspace,
    hashgrid_adam_step,
    hashgrid_backward,
    hashgrid_backward_noalloc,
    hashgrid_backward_workspace_size,
    hashgrid_debug_corners,
    forward_workspace,
    hashgrid_forward,
    hashgrid_forward_workspace_size,
    hashgrid_input_grad,
    hashgrid_mlp_backward,
    hashgrid_mlp_forward,
    hashgrid_mlp_workspace_size,
    hashgrid_input_grad_workspace_size,
    hashgrid_resolutions,
    hashgrid_tune,
    hashgrid_tune_get,
    load_library,
)
