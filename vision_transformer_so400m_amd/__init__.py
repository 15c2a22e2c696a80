"""MI355X (gfx950) SigLIP So400m/14 image encoder: a C-ABI HIP library
(libsiglip.so, include/siglip.h) and its thin Python binding."""
from ._lib import (  # noqa: F401
    EXPORTED, KCLASS, KERNEL_CLASSES, LIB_PATH, STAGE, STAGES, TEST_HOOKS, TEST_LIB_PATH, Model, SiglipError,
    attention, has_test_hooks, last_error, load_library, siglip_options, status_name, use_test_hooks,
    SIGLIP_OK, SIGLIP_E_INVALID_ARG, SIGLIP_E_BAD_BLOB, SIGLIP_E_UNSUPPORTED,
    SIGLIP_E_OUT_OF_MEMORY, SIGLIP_E_HIP,
)
