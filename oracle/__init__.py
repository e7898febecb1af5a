"""CPU oracle for hierarchical-layout evaluation and the layout-remapping copy.

TEST INFRASTRUCTURE ONLY.  Nothing in the library (the C ABI, the HIP kernels or
the Python binding in ``layout_remapping_copy_amd``) imports, links or calls this
package, and this package imports nothing from them.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

It is written from the three web pages the method is described on:

* [ThreadMap page] -- the article on CUTLASS 2.x ``PitchLinearStripminedThreadMap``
  at hotelren.com/news/5252042 (its sections 1.2, 2.2, 2.3, 3.3 are cited).
* [CuTe algebra page] -- "CUTE布局代数：GPU张量计算的内存优化革命"
  (jsqmd.com/news/768714), sections 2.1-2.3, 3.1-3.3, 4.2, 6.1.
* [print_layout page] -- "CUTLASS Layout可视化：从print_layout理解GPU内存映射与性能优化"
  (codechina.net/article/weixin_30702441/411096), sections 2.1-2.3, 3.1-3.2, 4.1-4.3, 5.2.

Every function is the plain definition, written for clarity, not speed (NumPy
vectorisation over the 1-D index is the only concession).  All arithmetic is on
Python ints or int64; element data are moved as opaque bytes.

Parity pins (values printed on the pages, closed forms, invariants, brute force)
live in ``tests/test_oracle.py`` and ``tests/golden/``.  No oracle function is
"parity unpinned".
"""

from .layout import (  # noqa: F401
    Layout,
    parse,
    fmt,
    flatten,
    top_modes,
    size,
    cosize,
    swizzle,
    eval_index,
    eval_indices,
    eval_coord,
    coalesce,
    compose,
    compose_table,
    right_inverse,
    right_inverse_fn,
    zipped_divide,
    slice_layout,
    complement,
    logical_divide,
    logical_product,
    blocked_product,
    is_injective,
    is_injective_bruteforce,
    injective_sufficient,
    max_common_vector,
    joint_flat,
    pitch_linear_offset,
    stripmined_offset,
    stripmined_layout,
    pitch_linear_layout,
    copy,
    copy_sampled_check,
    print_layout,
    bank_ways,
    lines_touched,
    lds_cycles,
    access_report,
    thread_offset_table,
    layout_grid,
)
