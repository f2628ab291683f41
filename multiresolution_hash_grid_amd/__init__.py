"""MI355X-native multiresolution hash-grid encoder.

The encoder runs in ``libhashgrid.so`` (HIP kernels for gfx950 behind the C
ABI of ``include/hashgrid.h``); ``hashgrid`` is its Python binding and
``inputs`` the seeded synthetic workload generator.
"""
from .hashgrid import (  # noqa: F401
    HashGridConfig,
    HashGridEncoder,
    HashGridError,
    HashGridFunction,
    abi_version,
    hashgrid_backward,
    hashgrid_debug_corners,
    hashgrid_forward,
    hashgrid_resolutions,
    hashgrid_tune,
    hashgrid_tune_get,
    load_library,
)
