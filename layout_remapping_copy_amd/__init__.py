"""Layout evaluation and layout-remapping copy on AMD MI355X (gfx950).

The work happens in ``lib/liblayout_remap.so`` (C ABI in ``include/layout_remap.h``:
C++ host algebra and hand-written HIP kernels); this package only marshals
arguments to it.  PyTorch provides device memory and streams.
"""

from .binding import (  # noqa: F401
    COPY_FORCE_PATH,
    COPY_ORDERED_ALIAS,
    COPY_WIDE_INDEX,
    PATH_ALIAS,
    PATH_DUAL,
    PATH_GENERIC,
    PATH_INTERLEAVE,
    PATH_STAGED,
    PATH_TRANSPOSE,
    PATH_TRANSPOSE_DIRECT,
    PATH_VECTOR,
    LIB_PATH,
    Layout,
    LayoutRemapError,
    access_check,
    LibraryNotBuilt,
    blocked_product,
    coalesce,
    complement,
    composition,
    copy_plan,
    header_symbols,
    is_injective,
    layout_copy,
    layout_eval,
    layout_eval_coords,
    layout_print,
    layout_print_table,
    lib,
    logical_divide,
    logical_product,
    max_common_vector,
    parse,
    right_inverse,
    thread_map,
    zipped_divide,
)
