"""Closed forms of the workload copies as NumPy reshapes, transposes and
takes.  TEST INFRASTRUCTURE ONLY.

Each function returns the expected destination bytes for a workload's source
bytes; they are the same results as ``oracle.copy`` (tests/test_oracle.py pins
each form against it at small sizes) but run in seconds at full size, so the GPU
tests can compare whole destination buffers, not only samples.
"""

from __future__ import annotations

import numpy as np


def transpose(src: np.ndarray, n: int) -> np.ndarray:
    """(n,n):(n,1) -> (n,n):(1,n): dst[j*n + i] = src[i*n + j]."""
    return np.ascontiguousarray(src.view(np.uint16).reshape(n, n).T).reshape(-1).view(np.uint8)


def retile(src: np.ndarray, n: int, tr: int = 128, tc: int = 64) -> np.ndarray:
    """Row-major n x n -> tr x tc tiles in row-major tile order, row-major inside a
    tile, then the 8-element (16-byte) chunk c of tile row r moves to c ^ (r % 8)
    (Swizzle<3,3,3> on bf16 offsets, [print_layout page, section 4.3])."""
    s = src.view(np.uint16).reshape(n // tr, tr, n // tc, tc).transpose(0, 2, 1, 3)
    tiles = s.reshape(-1, tr, tc // 8, 8)
    rows = np.arange(tr)[:, None]
    chunks = np.arange(tc // 8)[None, :]
    out = np.empty_like(tiles)
    out[:, rows, chunks ^ (rows % 8)] = tiles[:, rows, chunks]
    return out.reshape(-1).view(np.uint8)


def interleave(src: np.ndarray, b: int, h: int, s: int, d: int) -> np.ndarray:
    """(b,h,s,d) contiguous -> head pairs adjacent at stride 1 ([print_layout page,
    section 4.2]): dst[b][hp][s][d][hl] = src[b][2*hp + hl][s][d]."""
    x = src.view(np.uint16).reshape(b, h // 2, 2, s, d).transpose(0, 1, 3, 4, 2)
    return np.ascontiguousarray(x).reshape(-1).view(np.uint8)


def interleave_cm(src: np.ndarray, b: int, h: int, s: int, d: int) -> np.ndarray:
    """(b,h,s,d) contiguous -> dst[b][hp][d][s][hl] = src[b][2*hp + hl][s][d]: head
    pairs adjacent, (s, d) column-major inside a pair ([print_layout page, section
    4.2], its prose example read literally)."""
    x = src.view(np.uint16).reshape(b, h // 2, 2, s, d).transpose(0, 1, 4, 3, 2)
    return np.ascontiguousarray(x).reshape(-1).view(np.uint8)


_UINT = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def nhwc2nchw(src: np.ndarray, n: int, h: int, w: int, c: int, eb: int = 2) -> np.ndarray:
    """(n,h,w,c) contiguous -> (n,c,h,w) contiguous, elements of eb bytes."""
    x = src.view(_UINT[eb]).reshape(n, h, w, c).transpose(0, 3, 1, 2)
    return np.ascontiguousarray(x).reshape(-1).view(np.uint8)


def strided_copy(src: np.ndarray, shape, src_strides, dst: np.ndarray, dst_strides, eb: int) -> np.ndarray:
    """The copy between two flat (single-level, unswizzled) layouts of the same shape,
    as NumPy strided views: for every coordinate c, the eb-byte element at
    sum(c_i * dst_strides_i) of a copy of dst takes the one at sum(c_i * src_strides_i)
    of src (strides in elements).  Returns the new destination bytes."""
    item = np.dtype((np.void, eb))
    s = src.view(item)
    out = dst.copy()
    d = out.view(item)
    sv = np.lib.stride_tricks.as_strided(s, shape=tuple(shape), strides=tuple(eb * x for x in src_strides),
                                         writeable=False)
    dv = np.lib.stride_tricks.as_strided(d, shape=tuple(shape), strides=tuple(eb * x for x in dst_strides))
    dv[...] = sv
    return out


def transpose_batched(src: np.ndarray, batch: int, rows: int, cols: int, eb: int) -> np.ndarray:
    """batch row-major rows x cols matrices, one after another -> the same matrices
    transposed (cols x rows, row-major), elements of eb bytes moved as opaque bytes:
    dst[m][j][i] = src[m][i][j]."""
    x = src.reshape(batch, rows, cols, eb).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(x).reshape(-1)


def nchw2nhwc(src: np.ndarray, n: int, h: int, w: int, c: int, eb: int = 2) -> np.ndarray:
    """(n,c,h,w) contiguous -> (n,h,w,c) contiguous, elements of eb bytes."""
    x = src.view(_UINT[eb]).reshape(n, c, h, w).transpose(0, 2, 3, 1)
    return np.ascontiguousarray(x).reshape(-1).view(np.uint8)


def head_split(src: np.ndarray, b: int, s: int, h: int, d: int) -> np.ndarray:
    """(b,s,h,d) contiguous -> (b,h,s,d) contiguous, 2-byte elements."""
    x = src.view(np.uint16).reshape(b, s, h, d).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(x).reshape(-1).view(np.uint8)


def padtiles(src: np.ndarray, tiles: int) -> np.ndarray:
    """Per tile of 72 words: element k of the destination tile is word
    18*(k%4) + (k/4)%8 + 9*(k/32) of the source tile, i.e. the padded (8,8):(1,9)
    tile read through ((4,8),2):((16,1),8) ([CuTe algebra page, section 2.2])."""
    k = np.arange(64)
    table = 18 * (k % 4) + (k // 4) % 8 + 9 * (k // 32)
    s = src.view(np.uint32).reshape(tiles, 72)
    return np.ascontiguousarray(np.take(s, table, axis=1)).reshape(-1).view(np.uint8)


def shard_pack(src: np.ndarray, rows: int, cols: int, parts: int) -> np.ndarray:
    """Row block (rows, cols) row-major -> `parts` contiguous blocks, block j holding
    columns [j*w, (j+1)*w) transposed (w = cols / parts): dst[j][c][r] =
    src[r][j*w + c]."""
    x = src.view(np.uint16).reshape(rows, parts, cols // parts).transpose(1, 2, 0)
    return np.ascontiguousarray(x).reshape(-1).view(np.uint8)
