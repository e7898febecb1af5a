"""Seeded synthetic workloads for the layout-remapping copy.

This module only DESCRIBES inputs: layout texts, element sizes, buffer lengths and
seeded random bytes.  It holds none of the layout arithmetic (no evaluation,
composition or copying), so both the CPU oracle's tests and the HIP path's tests
and benchmark can share it without sharing the method.

The workloads (names follow the sizes they carry):

* ``tile8x8``     one 8x8 fp32 tile, column-major source, blocked (aliased)
                  destination ((4,2),(2,4)):((2,16),(1,8)).
* ``transpose``   fp16 8192x8192 row-major -> column-major, random 16-bit patterns.
* ``retile``      bf16 4096x4096 row-major -> 128x64 tiles in row-major tile order,
                  row-major inside a tile with Swizzle<3,3,3>.
* ``interleave``  bf16 (16,32,4096,128) contiguous -> heads paired at stride 1.
* ``interleave_cm`` the same tensor -> head pairs at stride 1 inside column-major
                  (s, d) tiles (the other reading of the interleaved layout).
* ``nhwc2nchw``   fp16 NHWC (128,56,56,256) -> NCHW.
* ``padtiles``    2**20 padded 8x8 fp32 tiles, source (8,8):(1,9) per tile read in
                  thread-value order ((4,8),2):((16,1),8), destination compact.
* ``rgb_nhwc2nchw`` fp16 NHWC (512,224,224,3) -> NCHW: three colour channels, so no
                  channel run reaches 16 bytes (the de-interleave).
* ``shard_pack``  the local pack of a transpose sharded by rows over 8 GPUs: one GPU's
                  1024 x 8192 fp16 row block -> 8 contiguous 1024 x 1024 blocks, block j
                  holding columns [1024 j, 1024 j + 1024) transposed (what GPU j receives).

Every workload takes a ``scale`` so tests can run the same structure small.
Destination buffers start filled with byte 0xA5 so untouched positions are checked.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

import numpy as np

SENTINEL_BYTE = 0xA5
PAD_WORD_F32 = 0x7FA5A5A5  # bit pattern written into the pad words of padded tiles


@dataclass
class Workload:
    name: str
    elem_bytes: int
    src_layout: str
    dst_layout: str
    src_elems: int           # source buffer length in elements
    dst_elems: int           # destination buffer length in elements
    seed: int
    values: str              # how the source bytes are drawn
    ordered_alias: bool = False
    extra_eval: List[str] = field(default_factory=list)  # layouts to evaluate on 0..size-1
    n_elems: int = 0          # logical elements copied (size of the layouts)
    note: str = ""


# ----------------------------------------------------------------------------
# Value generators (NumPy PCG64).  Floating-point values are rounded once, on the
# host, to the element type; afterwards every buffer is fixed bytes.
# ----------------------------------------------------------------------------
def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def gen_bits16(n: int, seed: int) -> np.ndarray:
    return _rng(seed).integers(0, 1 << 16, size=n, dtype=np.uint16).view(np.uint8)


def gen_uniform_f32(n: int, seed: int) -> np.ndarray:
    return _rng(seed).uniform(-1.0, 1.0, size=n).astype(np.float32).view(np.uint8)


def _normal_f32(n: int, seed: int) -> np.ndarray:
    return _rng(seed).standard_normal(size=n, dtype=np.float32)


def gen_normal_f16(n: int, seed: int) -> np.ndarray:
    return _normal_f32(n, seed).astype(np.float16).view(np.uint8)


def gen_normal_bf16(n: int, seed: int) -> np.ndarray:
    # round-to-nearest-even from fp32 to bf16 through torch on the CPU
    import torch

    x = torch.from_numpy(_normal_f32(n, seed))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8).copy()


def gen_bits(n_bytes: int, seed: int) -> np.ndarray:
    return _rng(seed).integers(0, 256, size=n_bytes, dtype=np.uint8)


_GEN: Dict[str, Callable[[int, int], np.ndarray]] = {
    "bits16": gen_bits16,
    "uniform_f32": gen_uniform_f32,
    "normal_f16": gen_normal_f16,
    "normal_bf16": gen_normal_bf16,
}


def make_src(w: Workload) -> np.ndarray:
    """Source buffer bytes for workload ``w`` (padded tiles get pad words)."""
    if w.name.startswith("padtiles"):
        n_tiles = w.src_elems // 72
        vals = gen_uniform_f32(n_tiles * 64, w.seed).view(np.uint32).reshape(n_tiles, 8, 8)
        buf = np.full((n_tiles, 8, 9), PAD_WORD_F32, dtype=np.uint32)
        buf[:, :, :8] = vals  # column j of a tile occupies words [9j, 9j+8); word 9j+8 is pad
        return buf.reshape(-1).view(np.uint8)
    return _GEN[w.values](w.src_elems, w.seed)


def make_dst(w: Workload) -> np.ndarray:
    return np.full(w.dst_elems * w.elem_bytes, SENTINEL_BYTE, dtype=np.uint8)


# ----------------------------------------------------------------------------
# Workload descriptions.  ``scale`` divides the large extents (keeping structure).
# ----------------------------------------------------------------------------
def tile8x8() -> Workload:
    return Workload(
        name="tile8x8", elem_bytes=4,
        src_layout="(8,8):(1,8)", dst_layout="((4,2),(2,4)):((2,16),(1,8))",
        src_elems=64, dst_elems=64, seed=1, values="uniform_f32", ordered_alias=True,
        extra_eval=["((4,8),2):((16,1),8)", "Sw<3,0,3> o (8,8):(8,1)"], n_elems=64,
        note="aliased destination: offsets 16..31 are written twice")


def transpose(n: int = 8192) -> Workload:
    return Workload(
        name=f"transpose{n}", elem_bytes=2,
        src_layout=f"({n},{n}):({n},1)", dst_layout=f"({n},{n}):(1,{n})",
        src_elems=n * n, dst_elems=n * n, seed=2, values="bits16", n_elems=n * n)


def retile(n: int = 4096, tr: int = 128, tc: int = 64) -> Workload:
    # row-major tile order over the (n/tr) x (n/tc) tile grid, row-major inside a tile
    tile = tr * tc
    return Workload(
        name=f"retile{n}", elem_bytes=2,
        src_layout=f"({n},{n}):({n},1)",
        dst_layout=(f"Sw<3,3,3> o (({tr},{n // tr}),({tc},{n // tc})):"
                    f"(({tc},{tile * (n // tc)}),(1,{tile}))"),
        src_elems=n * n, dst_elems=n * n, seed=3, values="normal_bf16", n_elems=n * n)


def interleave(b: int = 16, h: int = 32, s: int = 4096, d: int = 128) -> Workload:
    # logical (b, h, s, d); head h = hl + 2*hp; destination puts hl at stride 1
    sd = s * d
    return Workload(
        name=f"interleave{b}x{h}x{s}x{d}", elem_bytes=2,
        src_layout=f"({b},{h},{s},{d}):({h * sd},{sd},{d},1)",
        dst_layout=f"({b},(2,{h // 2}),{s},{d}):({h * sd},(1,{2 * sd}),{2 * d},2)",
        src_elems=b * h * sd, dst_elems=b * h * sd, seed=4, values="normal_bf16",
        n_elems=b * h * sd)


def interleave_cm(b: int = 16, h: int = 32, s: int = 4096, d: int = 128) -> Workload:
    # the column-major-inside reading of the interleaved pair: within a head pair,
    # (s, d) is stored column-major with the two heads adjacent, i.e. offset
    # 2*(s + S*d) + hl; logical (b, h, s, d) with h = hl + 2*hp
    sd = s * d
    return Workload(
        name=f"interleave_cm{b}x{h}x{s}x{d}", elem_bytes=2,
        src_layout=f"({b},{h},{s},{d}):({h * sd},{sd},{d},1)",
        dst_layout=f"({b},(2,{h // 2}),{s},{d}):({h * sd},(1,{2 * sd}),2,{2 * s})",
        src_elems=b * h * sd, dst_elems=b * h * sd, seed=7, values="normal_bf16",
        n_elems=b * h * sd)


def nhwc2nchw(n: int = 128, h: int = 56, w: int = 56, c: int = 256) -> Workload:
    hw = h * w
    return Workload(
        name=f"nhwc2nchw{n}x{h}x{w}x{c}", elem_bytes=2,
        src_layout=f"({n},{h},{w},{c}):({hw * c},{w * c},{c},1)",
        dst_layout=f"({n},{h},{w},{c}):({hw * c},{w},1,{hw})",
        src_elems=n * hw * c, dst_elems=n * hw * c, seed=5, values="normal_f16",
        n_elems=n * hw * c)


def padtiles(tiles: int = 1 << 20) -> Workload:
    # per tile: source (8,8):(1,9) composed with ((4,8),2):((16,1),8) is
    # ((4,8),2):((18,1),9); tiles 72 words apart; destination compact, 64 apart
    return Workload(
        name=f"padtiles{tiles}", elem_bytes=4,
        src_layout=f"((4,8),2,{tiles}):((18,1),9,72)",
        dst_layout=f"((4,8),2,{tiles}):((1,4),32,64)",
        src_elems=72 * tiles, dst_elems=64 * tiles, seed=6, values="uniform_f32",
        n_elems=64 * tiles)


def rgb_nhwc2nchw(n: int = 512, h: int = 224, w: int = 224, c: int = 3) -> Workload:
    wl = nhwc2nchw(n, h, w, c)
    wl.name = f"rgb_nhwc2nchw{n}x{h}x{w}x{c}"
    wl.seed = 9
    return wl


def shard_pack(rows: int = 1024, cols: int = 8192, parts: int = 8) -> Workload:
    # logical (r, c, j) with column j*w + c of the row block, w = cols / parts; block j
    # of the destination is contiguous, column-major over (r, c)
    w = cols // parts
    return Workload(
        name=f"shard_pack{rows}x{cols}/{parts}", elem_bytes=2,
        src_layout=f"({rows},{w},{parts}):({cols},1,{w})",
        dst_layout=f"({rows},{w},{parts}):(1,{rows},{rows * w})",
        src_elems=rows * cols, dst_elems=rows * cols, seed=8, values="bits16", n_elems=rows * cols)


def head_split(b: int = 16, s: int = 4096, h: int = 32, d: int = 128) -> Workload:
    # logical (b, s, h, d): a (batch, sequence, head, head-dim) tensor regrouped head by
    # head, (b, h, s, d); the head dimension stays contiguous on both sides (256-byte
    # atoms for bf16 d = 128)
    return Workload(
        name=f"head_split{b}x{s}x{h}x{d}", elem_bytes=2,
        src_layout=f"({b},{s},{h},{d}):({s * h * d},{h * d},{d},1)",
        dst_layout=f"({b},{s},{h},{d}):({h * s * d},{d},{s * d},1)",
        src_elems=b * s * h * d, dst_elems=b * s * h * d, seed=10, values="normal_bf16",
        n_elems=b * s * h * d)


FULL = {
    "tile8x8": tile8x8,
    "transpose": transpose,
    "retile": retile,
    "interleave": interleave,
    "interleave_cm": interleave_cm,
    "nhwc2nchw": nhwc2nchw,
    "padtiles": padtiles,
    "shard_pack": shard_pack,
    "rgb_nhwc2nchw": rgb_nhwc2nchw,
    "head_split": head_split,
}


def small(name: str) -> Workload:
    """Reduced sizes that still span several tiles and a ragged edge."""
    return {
        "tile8x8": tile8x8,
        "transpose": lambda: transpose(520),
        "retile": lambda: retile(512),
        "interleave": lambda: interleave(2, 4, 72, 128),
        "interleave_cm": lambda: interleave_cm(2, 4, 72, 136),
        "nhwc2nchw": lambda: nhwc2nchw(3, 7, 9, 40),
        "padtiles": lambda: padtiles(1000),
        "shard_pack": lambda: shard_pack(520, 2112, 8),
        "rgb_nhwc2nchw": lambda: rgb_nhwc2nchw(3, 17, 40, 3),
        "head_split": lambda: head_split(2, 70, 6, 128),
    }[name]()


def full(name: str) -> Workload:
    return FULL[name]()


def bytes_moved(w: Workload) -> int:
    """Algorithmic bytes: every element read once and written once."""
    return 2 * w.n_elems * w.elem_bytes
