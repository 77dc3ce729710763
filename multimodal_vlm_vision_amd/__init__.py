"""MI355X (gfx950) vision-tower forward: a HIP library behind a C ABI (include/vit.h).

The Python side is a thin ctypes binding (``binding``) plus torch-allocated
device buffers (``runtime``).  Import fails loudly when libvitmi.so is
missing: there is no CPU or PyTorch fallback.
"""

from .binding import (  # noqa: F401
    LIB_PATH,
    EmbeddingCache,
    Graph,
    Plan,
    VisionTower,
    VitError,
    header_symbols,
    load_library,
    make_config,
    resize_side,
    resize_u8,
)
