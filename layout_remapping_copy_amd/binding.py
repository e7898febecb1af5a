"""ctypes binding over liblayout_remap.so: argument marshalling only.

Every step of evaluation and copying runs in the C ABI (host algebra in C++,
device work in HIP kernels).  PyTorch supplies device memory and the current
stream; nothing here computes offsets or moves data.  When the shared library is
missing every call raises ``LibraryNotBuilt`` -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

LIB_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib")
LIB_PATH = os.path.join(LIB_DIR, "liblayout_remap.so")

MAX_LEAVES = 16

# lr_status
OK = 0
ERR_INVALID = -1
ERR_SIZE_MISMATCH = -2
ERR_BOUNDS = -3
ERR_OVERFLOW = -4
ERR_ALIAS = -5
ERR_NOT_REPRESENTABLE = -6
ERR_SWIZZLE = -7
ERR_ELEM_BYTES = -8
ERR_HIP = -9
ERR_PATH = -10
ERR_OVERLAP = -11
ERR_CAPACITY = -12

# lr_path
PATH_GENERIC = 0
PATH_VECTOR = 1
PATH_TRANSPOSE = 2
PATH_INTERLEAVE = 3
PATH_STAGED = 4
PATH_DUAL = 5
PATH_ALIAS = 6
PATH_TRANSPOSE_DIRECT = 7
PATH_DEINTERLEAVE = 8
PATH_BATCHED = 9
PATH_NAMES = {0: "generic", 1: "vector", 2: "transpose", 3: "interleave", 4: "staged", 5: "dual",
              6: "alias", 7: "transpose_direct", 8: "deinterleave", 9: "batched"}

# flags
COPY_ORDERED_ALIAS = 0x1
COPY_WIDE_INDEX = 0x2


def COPY_FORCE_PATH(p: int) -> int:
    return ((p + 1) & 0xFF) << 8


class lr_layout(ctypes.Structure):
    _fields_ = [
        ("nleaves", ctypes.c_int32),
        ("nmodes", ctypes.c_int32),
        ("shape", ctypes.c_int64 * MAX_LEAVES),
        ("stride", ctypes.c_int64 * MAX_LEAVES),
        ("mode_end", ctypes.c_int32 * MAX_LEAVES),
        ("swz_b", ctypes.c_int32),
        ("swz_m", ctypes.c_int32),
        ("swz_s", ctypes.c_int32),
    ]


class lr_plan(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("elem_bytes", ctypes.c_int32),
        ("vec_elems", ctypes.c_int32),
        ("wide", ctypes.c_int32),
        ("joint_rank", ctypes.c_int32),
        ("a_mode", ctypes.c_int32),
        ("b_mode", ctypes.c_int32),
        ("b2_mode", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("streaming", ctypes.c_int32),
        ("order", ctypes.c_int32),
        ("direct", ctypes.c_int32),
        ("load_policy", ctypes.c_int32),
        ("store_policy", ctypes.c_int32),
        ("vector_order", ctypes.c_int32),
        ("gather_chunks", ctypes.c_int32),
        ("pipeline_tiles", ctypes.c_int32),
        ("transpose_reads", ctypes.c_int32),
        ("batch_matrices", ctypes.c_int32),
        ("batch_swizzle", ctypes.c_int32 * 6),
        ("batch_order", ctypes.c_int32),
        ("tile_a", ctypes.c_int64),
        ("tile_b", ctypes.c_int64),
        ("grid", ctypes.c_int64),
        ("n_elems", ctypes.c_int64),
        ("blocks", ctypes.c_int64),
        ("ext", ctypes.c_int64 * (2 * MAX_LEAVES)),
        ("s_src", ctypes.c_int64 * (2 * MAX_LEAVES)),
        ("s_dst", ctypes.c_int64 * (2 * MAX_LEAVES)),
    ]


class lr_copy_tuning(ctypes.Structure):
    _fields_ = [
        ("load_policy", ctypes.c_int32),
        ("store_policy", ctypes.c_int32),
        ("units_per_lane", ctypes.c_int32),
        ("vector_order", ctypes.c_int32),
        ("interleave_form", ctypes.c_int32),
        ("tile_shape", ctypes.c_int32),
        ("tile_order", ctypes.c_int32),
        ("element_tiles", ctypes.c_int32),
        ("direct_loads", ctypes.c_int32),
        ("gather_chunks", ctypes.c_int32),
        ("pipeline_tiles", ctypes.c_int32),
        ("transpose_reads", ctypes.c_int32),
        ("chunk_bytes", ctypes.c_int32),
        ("batch_swizzle", ctypes.c_int32),
        ("batch_order", ctypes.c_int32),
        ("workgroup_lanes", ctypes.c_int32),
        ("transpose_blocks", ctypes.c_int32),
    ]


TUNING_FIELDS = tuple(k for k, _ in lr_copy_tuning._fields_)


def _tuning(tuning):
    """A dict of lr_copy_tuning fields (unnamed ones stay -1: the planner's choice)
    -> a pointer for the C call, or None."""
    if not tuning:
        return None
    t = lr_copy_tuning()
    lib().lr_copy_tuning_init(ctypes.byref(t))
    for k, v in tuning.items():
        if k not in TUNING_FIELDS:
            raise KeyError(f"unknown tuning field {k!r}")
        setattr(t, k, int(v))
    return ctypes.byref(t)


WAVE_LANES = 64


class lr_access_report(ctypes.Structure):
    _fields_ = [
        ("lanes", ctypes.c_int32),
        ("elem_bytes", ctypes.c_int32),
        ("banks", ctypes.c_int32),
        ("lanes_per_phase", ctypes.c_int32),
        ("line_bytes", ctypes.c_int32),
        ("phases", ctypes.c_int32),
        ("cycles", ctypes.c_int32),
        ("conflict_cycles", ctypes.c_int32),
        ("ways_max", ctypes.c_int32),
        ("bank_words", ctypes.c_int32 * WAVE_LANES),
        ("adjacent", ctypes.c_int32),
        ("first_gap", ctypes.c_int32),
        ("lines", ctypes.c_int64),
        ("min_lines", ctypes.c_int64),
        ("offsets", ctypes.c_int64 * WAVE_LANES),
    ]


class LibraryNotBuilt(RuntimeError):
    pass


class LayoutRemapError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})")


_P = ctypes.POINTER
_L = _P(lr_layout)
_SIGS = {
    "lr_layout_parse": (ctypes.c_int, [ctypes.c_char_p, _L]),
    "lr_layout_format": (ctypes.c_int, [_L, ctypes.c_char_p, ctypes.c_size_t]),
    "lr_layout_validate": (ctypes.c_int, [_L]),
    "lr_size": (ctypes.c_int, [_L, _P(ctypes.c_int64)]),
    "lr_cosize": (ctypes.c_int, [_L, _P(ctypes.c_int64)]),
    "lr_coalesce": (ctypes.c_int, [_L, _L]),
    "lr_composition": (ctypes.c_int, [_L, _L, _L]),
    "lr_right_inverse": (ctypes.c_int, [_L, _L]),
    "lr_zipped_divide": (ctypes.c_int, [_L, _P(ctypes.c_int64), ctypes.c_int32, _L]),
    "lr_complement": (ctypes.c_int, [_L, ctypes.c_int64, _L]),
    "lr_slice": (ctypes.c_int, [_L, _P(ctypes.c_int64), ctypes.c_int32, _L, _P(ctypes.c_int64)]),
    "lr_logical_divide": (ctypes.c_int, [_L, _L, _L]),
    "lr_logical_product": (ctypes.c_int, [_L, _L, _L]),
    "lr_blocked_product": (ctypes.c_int, [_L, _L, _L]),
    "lr_is_injective": (ctypes.c_int, [_L, _P(ctypes.c_int32)]),
    "lr_max_common_vector": (ctypes.c_int, [_L, _L, ctypes.c_size_t, _P(ctypes.c_int64)]),
    "lr_thread_map": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _L]),
    "lr_layout_print": (ctypes.c_int, [_L, ctypes.c_char_p, ctypes.c_size_t, _P(ctypes.c_size_t)]),
    "lr_layout_print_table": (ctypes.c_int, [_L, ctypes.c_int64, ctypes.c_char_p, ctypes.c_size_t,
                                             _P(ctypes.c_size_t)]),
    "lr_access_check": (ctypes.c_int, [_L, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, _P(lr_access_report)]),
    "lr_copy_plan": (ctypes.c_int, [_L, ctypes.c_int64, ctypes.c_size_t, _L, ctypes.c_int64, ctypes.c_size_t,
                                    ctypes.c_size_t, ctypes.c_uint32, _P(lr_plan)]),
    "lr_copy_tuning_init": (None, [_P(lr_copy_tuning)]),
    "lr_copy_plan_tuned": (ctypes.c_int, [_L, ctypes.c_int64, ctypes.c_size_t, _L, ctypes.c_int64, ctypes.c_size_t,
                                          ctypes.c_size_t, ctypes.c_uint32, _P(lr_copy_tuning), _P(lr_plan)]),
    "lr_layout_eval": (ctypes.c_int, [_L, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "lr_layout_eval_coords": (ctypes.c_int, [_L, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p]),
    "lr_layout_copy": (ctypes.c_int, [ctypes.c_void_p, _L, ctypes.c_int64, ctypes.c_void_p, _L, ctypes.c_int64,
                                      ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p]),
    "lr_layout_copy_tuned": (ctypes.c_int, [ctypes.c_void_p, _L, ctypes.c_int64, ctypes.c_void_p, _L, ctypes.c_int64,
                                            ctypes.c_size_t, ctypes.c_uint32, _P(lr_copy_tuning), ctypes.c_void_p]),
    "lr_layout_copy_count_writes": (ctypes.c_int, [ctypes.c_void_p, _L, ctypes.c_int64, ctypes.c_void_p, _L,
                                                   ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint32,
                                                   _P(lr_copy_tuning), ctypes.c_void_p, ctypes.c_void_p]),
    "lr_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "lr_last_hip_error": (ctypes.c_char_p, []),
    "lr_version": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """The loaded C library (raises LibraryNotBuilt if the .so is absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(f"{LIB_PATH} not found: run __graft_entry__.build() first")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def header_symbols(header_path: Optional[str] = None):
    """Names of the functions include/layout_remap.h declares."""
    if header_path is None:
        header_path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                                   "layout_remap.h")
    text = open(header_path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lr_\w+)\s*\(", text)) - {"lr_layout", "lr_plan"})


def strerror(code: int) -> str:
    return lib().lr_strerror(code).decode()


def _check(rc: int, what: str):
    if rc != OK:
        if rc == ERR_HIP:
            raise LayoutRemapError(rc, f"{what} [{lib().lr_last_hip_error().decode()}]")
        raise LayoutRemapError(rc, what)


# ---------------------------------------------------------------------------
# Layout handle
# ---------------------------------------------------------------------------
class Layout:
    """A descriptor (lr_layout) built and printed by the C library."""

    __slots__ = ("c",)

    def __init__(self, text_or_struct):
        if isinstance(text_or_struct, lr_layout):
            self.c = text_or_struct
        else:
            self.c = lr_layout()
            _check(lib().lr_layout_parse(str(text_or_struct).encode(), ctypes.byref(self.c)),
                   f"parse {text_or_struct!r}")

    def __str__(self):
        cap = 1024
        while True:
            buf = ctypes.create_string_buffer(cap)
            rc = lib().lr_layout_format(ctypes.byref(self.c), buf, len(buf))
            if rc != ERR_CAPACITY:
                _check(rc, "format")
                return buf.value.decode()
            cap *= 4

    __repr__ = __str__

    @property
    def leaves(self):
        return [(self.c.shape[i], self.c.stride[i]) for i in range(self.c.nleaves)]

    @property
    def mode_end(self):
        return [self.c.mode_end[i] for i in range(self.c.nmodes)]

    @property
    def swizzle(self):
        return (self.c.swz_b, self.c.swz_m, self.c.swz_s) if self.c.swz_b else None

    @property
    def size(self) -> int:
        n = ctypes.c_int64()
        _check(lib().lr_size(ctypes.byref(self.c), ctypes.byref(n)), "size")
        return n.value

    @property
    def cosize(self) -> int:
        n = ctypes.c_int64()
        _check(lib().lr_cosize(ctypes.byref(self.c), ctypes.byref(n)), "cosize")
        return n.value


def _as_layout(x) -> Layout:
    return x if isinstance(x, Layout) else Layout(x)


def parse(text: str) -> Layout:
    return Layout(text)


def layout_parse(text: str) -> Layout:
    """lr_layout_parse."""
    return Layout(text)


def layout_format(L) -> str:
    """lr_layout_format."""
    return str(_as_layout(L))


def layout_validate(L) -> None:
    """lr_layout_validate: raises LayoutRemapError for a bad descriptor."""
    _check(lib().lr_layout_validate(ctypes.byref(_as_layout(L).c)), "validate")


def size(L) -> int:
    """lr_size."""
    return _as_layout(L).size


def cosize(L) -> int:
    """lr_cosize."""
    return _as_layout(L).cosize


def last_hip_error() -> str:
    """lr_last_hip_error: text of the last HIP error on this thread."""
    return lib().lr_last_hip_error().decode()


def version() -> str:
    """lr_version."""
    return lib().lr_version().decode()


def coalesce(L) -> Layout:
    out = lr_layout()
    _check(lib().lr_coalesce(ctypes.byref(_as_layout(L).c), ctypes.byref(out)), "coalesce")
    return Layout(out)


def composition(A, B) -> Layout:
    out = lr_layout()
    _check(lib().lr_composition(ctypes.byref(_as_layout(A).c), ctypes.byref(_as_layout(B).c), ctypes.byref(out)),
           "composition")
    return Layout(out)


def right_inverse(L) -> Layout:
    out = lr_layout()
    _check(lib().lr_right_inverse(ctypes.byref(_as_layout(L).c), ctypes.byref(out)), "right_inverse")
    return Layout(out)


def zipped_divide(L, tiler: Sequence[int]) -> Layout:
    out = lr_layout()
    arr = (ctypes.c_int64 * max(1, len(tiler)))(*tiler)
    _check(lib().lr_zipped_divide(ctypes.byref(_as_layout(L).c), arr, len(tiler), ctypes.byref(out)),
           "zipped_divide")
    return Layout(out)


def complement(A, M: int) -> Layout:
    out = lr_layout()
    _check(lib().lr_complement(ctypes.byref(_as_layout(A).c), M, ctypes.byref(out)), "complement")
    return Layout(out)


def slice(L, coord: Sequence[int]):
    """lr_slice: (the layout of the kept coordinates, the offset of the fixed ones).
    coord: one entry per top-level mode or per leaf, -1 (or None) keeping it."""
    L = _as_layout(L)
    vals = [-1 if c is None else int(c) for c in coord]
    arr = (ctypes.c_int64 * max(1, len(vals)))(*vals)
    out = lr_layout()
    off = ctypes.c_int64()
    _check(lib().lr_slice(ctypes.byref(L.c), arr, len(vals), ctypes.byref(out), ctypes.byref(off)), "slice")
    return Layout(out), off.value


def _binary(name: str, A, B) -> Layout:
    out = lr_layout()
    _check(getattr(lib(), name)(ctypes.byref(_as_layout(A).c), ctypes.byref(_as_layout(B).c), ctypes.byref(out)),
           name)
    return Layout(out)


def logical_divide(A, B) -> Layout:
    return _binary("lr_logical_divide", A, B)


def logical_product(A, B) -> Layout:
    return _binary("lr_logical_product", A, B)


def blocked_product(A, B) -> Layout:
    return _binary("lr_blocked_product", A, B)


def is_injective(L) -> bool:
    r = ctypes.c_int32()
    _check(lib().lr_is_injective(ctypes.byref(_as_layout(L).c), ctypes.byref(r)), "is_injective")
    return bool(r.value)


def max_common_vector(Ls, Ld, elem_bytes: int) -> int:
    r = ctypes.c_int64()
    _check(lib().lr_max_common_vector(ctypes.byref(_as_layout(Ls).c), ctypes.byref(_as_layout(Ld).c), elem_bytes,
                                      ctypes.byref(r)), "max_common_vector")
    return r.value


def thread_map(pitch: int, strips: int, krow: int, threads: int) -> Layout:
    out = lr_layout()
    _check(lib().lr_thread_map(pitch, strips, krow, threads, ctypes.byref(out)), "thread_map")
    return Layout(out)


def _print_text(fn, what, *args) -> str:
    need = ctypes.c_size_t()
    rc = fn(*args, None, 0, ctypes.byref(need))
    if rc != ERR_CAPACITY:
        _check(rc, what)
    buf = ctypes.create_string_buffer(need.value)
    _check(fn(*args, buf, need.value, ctypes.byref(need)), what)
    return buf.value.decode()


def layout_print(L) -> str:
    """Grid of a two-mode layout: rows over mode 0, columns over mode 1."""
    return _print_text(lib().lr_layout_print, "layout_print", ctypes.byref(_as_layout(L).c))


def layout_print_table(L, n: int) -> str:
    """'thread t -> offset L(t)' for t < n."""
    return _print_text(lib().lr_layout_print_table, "layout_print_table", ctypes.byref(_as_layout(L).c), n)


LDS_CUSTOM = 0
LDS_GFX950_READ = 1
LDS_GFX950_WRITE = 2


def access_check(L, elem_bytes: int, lanes: int = WAVE_LANES, op: str = "read", banks: int = 0,
                 lanes_per_phase: int = 0, line_bytes: int = 0) -> dict:
    """Bank cycles, adjacency and cache lines of one wavefront accessing L(0..lanes-1).
    op "read"/"write" selects the gfx950 LDS model; op "custom" uses banks and
    lanes_per_phase."""
    model = {"read": LDS_GFX950_READ, "write": LDS_GFX950_WRITE, "custom": LDS_CUSTOM}[op]
    r = lr_access_report()
    _check(lib().lr_access_check(ctypes.byref(_as_layout(L).c), elem_bytes, lanes, model, banks, lanes_per_phase,
                                 line_bytes, ctypes.byref(r)), "access_check")
    out = {k: getattr(r, k) for k, _ in lr_access_report._fields_ if k not in ("bank_words", "offsets")}
    out["bank_words"] = list(r.bank_words[:r.banks])
    out["offsets"] = list(r.offsets[:r.lanes])
    out["adjacent"] = bool(r.adjacent)
    return out


def copy_plan(Ls, src_capacity: int, Ld, dst_capacity: int, elem_bytes: int, flags: int = 0,
              src_align: int = 16, dst_align: int = 16, tuning: Optional[dict] = None) -> dict:
    """The plan lr_layout_copy would launch (host only).  ``tuning``: a dict of
    lr_copy_tuning fields overriding the planner's launch choices."""
    p = lr_plan()
    _check(lib().lr_copy_plan_tuned(ctypes.byref(_as_layout(Ls).c), src_capacity, src_align,
                                    ctypes.byref(_as_layout(Ld).c), dst_capacity, dst_align, elem_bytes, flags,
                                    _tuning(tuning), ctypes.byref(p)), "copy_plan")
    r = p.joint_rank
    return {
        "path": PATH_NAMES[p.path], "elem_bytes": p.elem_bytes, "vec_elems": p.vec_elems, "wide": bool(p.wide),
        "a_mode": p.a_mode, "b_mode": p.b_mode, "b2_mode": p.b2_mode, "block": p.block,
        "streaming": bool(p.streaming), "order": p.order, "direct": bool(p.direct),
        "load_policy": p.load_policy, "store_policy": p.store_policy,
        "vector_order": p.vector_order, "gather_chunks": p.gather_chunks, "pipeline_tiles": p.pipeline_tiles,
        "transpose_reads": bool(p.transpose_reads),
        "batch_matrices": p.batch_matrices, "batch_swizzle": tuple(p.batch_swizzle), "batch_order": p.batch_order,
        "tile_a": p.tile_a, "tile_b": p.tile_b,
        "grid": p.grid, "n_elems": p.n_elems, "blocks": p.blocks,
        "joint": [(p.ext[i], p.s_src[i], p.s_dst[i]) for i in range(r)],
    }


# ---------------------------------------------------------------------------
# Device entry points (torch tensors for memory and stream only)
# ---------------------------------------------------------------------------
def _torch():
    import torch

    return torch


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _device_tensor(t, what: str):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def layout_eval(L, idx=None, n: Optional[int] = None, device="cuda", stream=None):
    """Offsets of L at 1-D indices (an int64 GPU tensor) or at 0..n-1."""
    torch = _torch()
    L = _as_layout(L)
    if idx is not None:
        _device_tensor(idx, "idx")
        if idx.dtype != torch.int64:
            raise TypeError("idx must be int64")
        n = idx.numel()
        dev = idx.device
    else:
        if n is None:
            n = L.size
        dev = torch.device(device)
    out = torch.empty(n, dtype=torch.int64, device=dev)
    _check(lib().lr_layout_eval(ctypes.byref(L.c), idx.data_ptr() if idx is not None else None, n,
                                out.data_ptr(), _stream_ptr(stream)), "layout_eval")
    return out


def layout_eval_coords(L, coords, stream=None):
    """Offsets of L at coordinates: coords is an (n, ncols) int64 GPU tensor with
    ncols == number of top-level modes or == number of leaves."""
    torch = _torch()
    L = _as_layout(L)
    _device_tensor(coords, "coords")
    if coords.dtype != torch.int64 or coords.dim() != 2:
        raise TypeError("coords must be a 2-D int64 tensor")
    n, ncols = coords.shape
    out = torch.empty(n, dtype=torch.int64, device=coords.device)
    _check(lib().lr_layout_eval_coords(ctypes.byref(L.c), coords.data_ptr(), n, ncols, out.data_ptr(),
                                       _stream_ptr(stream)), "layout_eval_coords")
    return out


def layout_copy(src, Ls, dst, Ld, elem_bytes: Optional[int] = None, flags: int = 0, stream=None,
                tuning: Optional[dict] = None):
    """dst[Ld(k)] = src[Ls(k)] for every k, on the GPU; src and dst are contiguous
    GPU tensors viewed as flat element buffers of ``elem_bytes`` bytes.  ``tuning``:
    a dict of lr_copy_tuning fields overriding the planner's launch choices (the
    result is the same bytes)."""
    _device_tensor(src, "src")
    _device_tensor(dst, "dst")
    if src.device != dst.device:
        raise ValueError("src and dst must be on the same device")
    Ls, Ld = _as_layout(Ls), _as_layout(Ld)
    eb = elem_bytes if elem_bytes is not None else src.element_size()
    sb = src.numel() * src.element_size()
    db = dst.numel() * dst.element_size()
    if sb % eb or db % eb:
        raise ValueError("buffer sizes are not multiples of elem_bytes")
    if tuning:
        rc = lib().lr_layout_copy_tuned(src.data_ptr(), ctypes.byref(Ls.c), sb // eb, dst.data_ptr(),
                                        ctypes.byref(Ld.c), db // eb, eb, flags, _tuning(tuning), _stream_ptr(stream))
    else:
        rc = lib().lr_layout_copy(src.data_ptr(), ctypes.byref(Ls.c), sb // eb, dst.data_ptr(), ctypes.byref(Ld.c),
                                  db // eb, eb, flags, _stream_ptr(stream))
    _check(rc, "layout_copy")
    return dst


def copy_tuning_init() -> dict:
    """lr_copy_tuning_init: every override at -1 (the planner's choices), as a dict."""
    t = lr_copy_tuning()
    lib().lr_copy_tuning_init(ctypes.byref(t))
    return {k: getattr(t, k) for k in TUNING_FIELDS}


def copy_plan_tuned(Ls, src_capacity: int, Ld, dst_capacity: int, elem_bytes: int, tuning: dict, flags: int = 0,
                    src_align: int = 16, dst_align: int = 16) -> dict:
    """lr_copy_plan_tuned: copy_plan with overrides."""
    return copy_plan(Ls, src_capacity, Ld, dst_capacity, elem_bytes, flags, src_align, dst_align, tuning=tuning)


def layout_copy_tuned(src, Ls, dst, Ld, tuning: dict, elem_bytes: Optional[int] = None, flags: int = 0, stream=None):
    """lr_layout_copy_tuned: layout_copy with overrides."""
    return layout_copy(src, Ls, dst, Ld, elem_bytes, flags, stream, tuning=tuning)


def layout_copy_count_writes(src, Ls, dst, Ld, counts, elem_bytes: Optional[int] = None, flags: int = 0,
                             stream=None, tuning: Optional[dict] = None):
    """lr_layout_copy_count_writes: layout_copy that also adds, in the int32 GPU
    tensor ``counts`` (one entry per destination element, zeroed by the caller),
    one per store the kernels make to each destination element."""
    torch = _torch()
    _device_tensor(src, "src")
    _device_tensor(dst, "dst")
    _device_tensor(counts, "counts")
    if counts.dtype != torch.int32:
        raise TypeError("counts must be int32")
    Ls, Ld = _as_layout(Ls), _as_layout(Ld)
    eb = elem_bytes if elem_bytes is not None else src.element_size()
    sb = src.numel() * src.element_size()
    db = dst.numel() * dst.element_size()
    if sb % eb or db % eb:
        raise ValueError("buffer sizes are not multiples of elem_bytes")
    if counts.numel() < db // eb:
        raise ValueError("counts needs one entry per destination element")
    _check(lib().lr_layout_copy_count_writes(src.data_ptr(), ctypes.byref(Ls.c), sb // eb, dst.data_ptr(),
                                             ctypes.byref(Ld.c), db // eb, eb, flags, _tuning(tuning),
                                             counts.data_ptr(), _stream_ptr(stream)), "layout_copy_count_writes")
    return counts
