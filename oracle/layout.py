"""Plain definitions of hierarchical layouts and the layout-remapping copy.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Short page names used in
the citations below:

* [ThreadMap page]      CUTLASS 2.x PitchLinearStripminedThreadMap article (hotelren.com/news/5252042)
* [CuTe algebra page]   "CUTE布局代数：GPU张量计算的内存优化革命" (jsqmd.com/news/768714)
* [print_layout page]   "CUTLASS Layout可视化：从print_layout理解GPU内存映射与性能优化"
                        (codechina.net/article/weixin_30702441/411096)

Readings taken where the pages are silent or garbled (each one is also tested):

* A 1-D index (and a thread id) is split into coordinates colexicographically:
  the first leaf varies fastest.  The ThreadMap page splits a thread id with the
  contiguous part ``tid % Pitch`` first (sections 1.2 and 2.2), and the CuTe
  algebra page calls (8,8):(1,8) column-major with neighbours adjacent down a
  column (section 2.1).
* ``Swizzle<B,M,S>`` acts on the final element offset:
  ``o ^ ((o >> S) & (((1 << B) - 1) << M))``; with S >= B it is an involution.
  With B=3, M=0, S=3 on (8,8):(8,1) it gives the print_layout page's formula
  ``row*8 + (col ^ row)`` (section 4.3); the rows that page prints below the
  formula contradict it, and the formula is taken.
* Composition ``A o B`` is ``c -> A(B(c))`` with B's integer result used as a 1-D
  index into A; A is coalesced first and its last leaf is extended without bound
  when ``B(c) >= size(A)``.
* For an aliased (non-injective) destination the copy is the sequential loop over
  the index in increasing order, so the greatest index writing an offset wins.
"""

from __future__ import annotations

import re
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple, Union

import math

import numpy as np

Nested = Union[int, tuple]


# ----------------------------------------------------------------------------
# Layout value: a congruent pair of nested integer tuples plus an optional swizzle.
# [CuTe algebra page, section 2.1]: a layout maps logical coordinates to offsets.
# [print_layout page, sections 2.1 and 3.2]: shape gives the extents, stride the
# offset step of each mode; "(4,2):(_2,_1)" is the printed form.
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Layout:
    shape: Nested
    stride: Nested
    swz: Optional[Tuple[int, int, int]] = None  # (B, M, S) or None

    def __post_init__(self):
        _check_congruent(self.shape, self.stride)
        for n in _leaves(self.shape):
            if n < 1:
                raise ValueError("extent must be >= 1")
        if self.swz is not None:
            b, m, s = self.swz
            if b < 0 or m < 0 or s < b:
                raise ValueError("swizzle needs B >= 0, M >= 0, S >= B")

    def __call__(self, *coord):
        if len(coord) == 1 and isinstance(coord[0], int):
            return eval_index(self, coord[0])
        return eval_coord(self, coord if len(coord) > 1 else coord[0])

    def __str__(self):
        return fmt(self)


def _leaves(t: Nested):
    if isinstance(t, int):
        return [t]
    out = []
    for x in t:
        out.extend(_leaves(x))
    return out


def _check_congruent(a: Nested, b: Nested):
    if isinstance(a, int) != isinstance(b, int):
        raise ValueError("shape and stride are not congruent")
    if isinstance(a, tuple):
        if len(a) != len(b):
            raise ValueError("shape and stride are not congruent")
        for x, y in zip(a, b):
            _check_congruent(x, y)


# ----------------------------------------------------------------------------
# Text form.  [print_layout page, section 3.2]: "(shape):(stride)" with optional
# compile-time markers "_"; a swizzle is written "Sw<B,M,S> o layout".
# ----------------------------------------------------------------------------
_TOKEN = re.compile(r"\s*(Swizzle|Sw|[()<>,:]|o|∘|_?-?\d+)")


def _tokens(text: str):
    pos, out = 0, []
    text = text.strip()
    while pos < len(text):
        m = _TOKEN.match(text, pos)
        if not m:
            raise ValueError(f"bad layout text at {pos}: {text!r}")
        out.append(m.group(1))
        pos = m.end()
        while pos < len(text) and text[pos].isspace():
            pos += 1
    return out


def parse(text: str) -> Layout:
    toks = _tokens(text)
    i = 0

    def peek():
        return toks[i] if i < len(toks) else None

    def take(expect=None):
        nonlocal i
        t = peek()
        if t is None or (expect is not None and t != expect):
            raise ValueError(f"expected {expect!r}, got {t!r} in {text!r}")
        i += 1
        return t

    def integer():
        t = take()
        if not re.fullmatch(r"_?-?\d+", t):
            raise ValueError(f"expected integer, got {t!r}")
        return int(t.lstrip("_"))

    def tup():
        if peek() == "(":
            take("(")
            items = [tup()]
            while peek() == ",":
                take(",")
                items.append(tup())
            take(")")
            return tuple(items)
        return integer()

    swz = None
    if peek() in ("Sw", "Swizzle"):
        take()
        take("<")
        b = integer()
        take(",")
        m = integer()
        take(",")
        s = integer()
        take(">")
        if peek() not in ("o", "∘"):
            raise ValueError("expected 'o' after swizzle")
        take()
        swz = (b, m, s)
    shape = tup()
    take(":")
    stride = tup()
    if peek() is not None:
        raise ValueError(f"trailing text in {text!r}")
    if swz is not None and swz[0] == 0:
        swz = None
    return Layout(shape, stride, swz)


def _fmt_t(t: Nested) -> str:
    if isinstance(t, int):
        return str(t)
    return "(" + ",".join(_fmt_t(x) for x in t) + ")"


def fmt(L: Layout) -> str:
    body = f"{_fmt_t(L.shape)}:{_fmt_t(L.stride)}"
    if L.swz is not None:
        return f"Sw<{L.swz[0]},{L.swz[1]},{L.swz[2]}> o {body}"
    return body


# ----------------------------------------------------------------------------
# Structure.  [CuTe algebra page, section 2.1] and [print_layout page, section
# 2.1]: a layout is shape and stride, one extent and one step per mode; its size
# is the number of coordinates, the product of the extents.
# ----------------------------------------------------------------------------
def flatten(L: Layout):
    """Leaves depth-first, left to right, as a list of (extent, stride)."""
    return list(zip(_leaves(L.shape), _leaves(L.stride)))


def top_modes(L: Layout):
    """Top-level modes as sub-layouts (a rank-0 shape is one mode)."""
    if isinstance(L.shape, int):
        return [Layout(L.shape, L.stride)]
    return [Layout(s, d) for s, d in zip(L.shape, L.stride)]


def size(L: Layout) -> int:
    p = 1
    for n, _ in flatten(L):
        p *= n
    return p


def swizzle(o, swz):
    """[print_layout page, section 4.3]: XOR the B bits at [M+S, M+S+B) into the
    bits at [M, M+B).  Works on Python ints and on int64 NumPy arrays."""
    if swz is None:
        return o
    b, m, s = swz
    mask = ((1 << b) - 1) << m
    return o ^ ((o >> s) & mask)


def eval_index(L: Layout, k: int) -> int:
    """1-D index -> offset: colex digits, then sum of digit*stride, then swizzle.
    [print_layout page, section 2.1] gives offset = sum of coordinate * stride."""
    if not 0 <= k < size(L):
        raise IndexError(k)
    off = 0
    for n, d in flatten(L):
        off += (k % n) * d
        k //= n
    return swizzle(off, L.swz)


def eval_indices(L: Layout, ks: np.ndarray) -> np.ndarray:
    """Vectorised ``eval_index`` over an int64 array of indices."""
    ks = np.asarray(ks, dtype=np.int64).copy()
    off = np.zeros_like(ks)
    for n, d in flatten(L):
        off += (ks % n) * d
        ks //= n
    return swizzle(off, L.swz)


def _crd2off(c, shape, stride) -> int:
    if isinstance(c, int):
        # an integer at any level is split colexicographically over that sub-shape
        leaves = list(zip(_leaves(shape), _leaves(stride)))
        total = 1
        for n, _ in leaves:
            total *= n
        if not 0 <= c < total:
            raise IndexError(c)
        off = 0
        for n, d in leaves:
            off += (c % n) * d
            c //= n
        return off
    if isinstance(shape, int) or len(c) != len(shape):
        raise ValueError("coordinate not congruent with shape")
    return sum(_crd2off(ci, si, di) for ci, si, di in zip(c, shape, stride))


def eval_coord(L: Layout, coord) -> int:
    """Offset of a (possibly nested) coordinate.  [print_layout page, section 6.3]:
    a layout is called with two integers or with one coordinate object; an integer
    given for a nested mode is split colexicographically inside that mode."""
    if isinstance(L.shape, int):
        if isinstance(coord, tuple) and len(coord) == 1:
            coord = coord[0]
        return swizzle(_crd2off(coord, L.shape, L.stride), L.swz)
    return swizzle(_crd2off(tuple(coord), L.shape, L.stride), L.swz)


def _max_offset_linear(L: Layout) -> int:
    return sum((n - 1) * d for n, d in flatten(L))


def cosize(L: Layout) -> int:
    """Exact max offset + 1 (brute force when swizzled).  Strides are >= 0."""
    if L.swz is None:
        return _max_offset_linear(L) + 1
    return int(eval_indices(L, np.arange(size(L), dtype=np.int64)).max()) + 1


def layout_grid(L: Layout):
    """[print_layout page, sections 2.3 and 3.3]: outer loop over mode 0, inner loop
    over mode 1, each cell the offset of (row, col).  Rank-2 layouts only."""
    modes = top_modes(L)
    if len(modes) != 2:
        raise ValueError("grid needs exactly two top-level modes")
    r, c = size(modes[0]), size(modes[1])
    return [[eval_coord(L, (i, j)) for j in range(c)] for i in range(r)]


def print_layout(L: Layout) -> str:
    rows = layout_grid(L)
    width = max(len(str(v)) for row in rows for v in row)
    lines = [fmt(L)]
    for row in rows:
        lines.append(" ".join(str(v).rjust(width) for v in row))
    return "\n".join(lines)


# ----------------------------------------------------------------------------
# Access-pattern checks.  [print_layout page, sections 4.3, 5.2 and 6.4]: shared
# memory is split into banks, accesses by one warp to different addresses in the
# same bank are serialised (the same address is broadcast), padding a row by one
# element or an XOR swizzle spreads a column over the banks; adjacent threads
# should touch adjacent addresses so a warp's accesses fall in few cache lines.
# Lane t accesses element L(t) (elem_bytes bytes).
# ----------------------------------------------------------------------------
def bank_ways(L: Layout, elem_bytes: int, lanes: int = 32, banks: int = 32, bank_bytes: int = 4) -> int:
    """Largest number of distinct bank words one bank must serve for the access
    of lanes 0..lanes-1 (1 means conflict-free)."""
    per_bank = {}
    for t in range(lanes):
        a = eval_index(L, t) * elem_bytes
        for w in range(a // bank_bytes, (a + elem_bytes - 1) // bank_bytes + 1):
            per_bank.setdefault(w % banks, set()).add(w)
    return max(len(v) for v in per_bank.values())


def lines_touched(L: Layout, elem_bytes: int, lanes: int = 64, line_bytes: int = 128) -> int:
    """Distinct cache lines the access of lanes 0..lanes-1 touches."""
    lines = set()
    for t in range(lanes):
        a = eval_index(L, t) * elem_bytes
        lines.update(range(a // line_bytes, (a + elem_bytes - 1) // line_bytes + 1))
    return len(lines)


def lds_cycles(L: Layout, elem_bytes: int, lanes: int, banks: int, lanes_per_phase: int):
    """One wavefront access served in phases of lanes_per_phase consecutive lanes;
    each phase costs the bank_ways of its own lanes.  Returns (cycles, phases,
    worst ways, distinct words per bank in the first worst phase)."""
    cycles, worst, hist, phases = 0, 0, None, 0
    for p in range(0, lanes, lanes_per_phase):
        per_bank = {}
        for t in range(p, min(lanes, p + lanes_per_phase)):
            a = eval_index(L, t) * elem_bytes
            for w in range(a // 4, (a + elem_bytes - 1) // 4 + 1):
                per_bank.setdefault(w % banks, set()).add(w)
        ways = max(len(v) for v in per_bank.values())
        cycles += ways
        phases += 1
        if ways > worst:
            worst = ways
            hist = [len(per_bank.get(b, ())) for b in range(banks)]
    return cycles, phases, worst, hist


def access_report(L: Layout, elem_bytes: int, lanes: int, banks: int, lanes_per_phase: int,
                  line_bytes: int = 128) -> dict:
    """[print_layout page, section 6.4]: the two checks on a candidate layout, for
    lane t accessing element L(t): are consecutive lanes on consecutive offsets, and
    how evenly do the lanes spread over the banks; plus the cache lines touched."""
    offs = [eval_index(L, t) for t in range(lanes)]
    cyc, ph, worst, hist = lds_cycles(L, elem_bytes, lanes, banks, lanes_per_phase)
    gap = next((t for t in range(lanes - 1) if offs[t + 1] != offs[t] + 1), -1)
    byts = {o * elem_bytes + i for o in offs for i in range(elem_bytes)}
    return {"offsets": offs, "cycles": cyc, "phases": ph, "ways_max": worst,
            "conflict_cycles": cyc - ph, "bank_words": hist,
            "lines": lines_touched(L, elem_bytes, lanes, line_bytes),
            "min_lines": -(-len(byts) // line_bytes),
            "adjacent": gap < 0, "first_gap": gap}


def thread_offset_table(L: Layout, n: int) -> str:
    """[ThreadMap page, section 5.3]: the thread-to-offset table, one line per
    thread, numbers right-aligned to the widest entry."""
    offs = [eval_index(L, t) for t in range(n)]
    wt = len(str(n - 1))
    wo = max(len(str(o)) for o in offs)
    return "\n".join(f"thread {t:>{wt}} -> offset {o:>{wo}}" for t, o in enumerate(offs))


# ----------------------------------------------------------------------------
# Coalesce: the same function of the 1-D index on [0, size) with extent-1 leaves
# dropped and neighbours merged whenever stride[i+1] == extent[i] * stride[i].
# ----------------------------------------------------------------------------
def _coalesce_leaves(leaves):
    out = []
    for n, d in leaves:
        if n == 1:
            continue
        if out and d == out[-1][0] * out[-1][1]:
            out[-1] = (out[-1][0] * n, out[-1][1])
        else:
            out.append((n, d))
    return out


def _from_leaves(leaves, swz=None) -> Layout:
    if not leaves:
        return Layout(1, 0, swz)
    if len(leaves) == 1:
        return Layout(leaves[0][0], leaves[0][1], swz)
    return Layout(tuple(n for n, _ in leaves), tuple(d for _, d in leaves), swz)


def coalesce(L: Layout) -> Layout:
    return _from_leaves(_coalesce_leaves(flatten(L)), L.swz)


# ----------------------------------------------------------------------------
# Composition.  [CuTe algebra page, section 2.2]: R = A o B reshapes or re-orders
# access while the data stay put; with a padded A the padding is skipped.
# ----------------------------------------------------------------------------
class NotRepresentable(Exception):
    pass


def _compose_leaf(a_leaves, n: int, s: int):
    """Leaves of k -> A(s*k), k in [0, n), against coalesced A leaves, the last of
    which is unbounded.  Raises NotRepresentable when a divisibility fails."""
    if n == 1:
        return [(1, 0)]
    if s == 0:
        return [(n, 0)]
    leaves = list(a_leaves) if a_leaves else [(1, 0)]
    # 1) divide the stride out of A's leading extents
    rest = s
    i = 0
    while True:
        ext, d = leaves[i]
        last = i == len(leaves) - 1
        if last:
            cur = (None, d * rest)  # unbounded
            break
        if rest % ext == 0:
            rest //= ext
            i += 1
            continue
        if ext % rest == 0:
            cur = (ext // rest, d * rest)
            break
        raise NotRepresentable(f"stride {s} does not divide through extent {ext}")
    # 2) take n elements from the remaining leaves
    out = []
    remaining = n
    while remaining > 1:
        ext, d = cur
        if ext is None:
            out.append((remaining, d))
            remaining = 1
            break
        if remaining % ext == 0:
            if ext > 1:
                out.append((ext, d))
            remaining //= ext
            i += 1
            if remaining == 1:
                break
            nxt = leaves[i]
            cur = (None if i == len(leaves) - 1 else nxt[0], nxt[1])
            continue
        if ext % remaining == 0:
            out.append((remaining, d))
            remaining = 1
            break
        raise NotRepresentable(f"extent {remaining} does not divide extent {ext}")
    return out


def _map_shape(shape, stride, fn):
    if isinstance(shape, int):
        return fn(shape, stride)
    pairs = [_map_shape(s, d, fn) for s, d in zip(shape, stride)]
    return tuple(p[0] for p in pairs), tuple(p[1] for p in pairs)


def compose(A: Layout, B: Layout) -> Layout:
    """Closed form of A o B with B's shape; raises NotRepresentable."""
    a_leaves = _coalesce_leaves(flatten(A))
    if B.swz is not None:
        # only an unswizzled A that is the identity (n:1, extended without bound)
        # lets B's swizzle pass through unchanged
        if A.swz is None and len(a_leaves) == 1 and a_leaves[0][1] == 1:
            return B
        raise NotRepresentable("swizzled right operand")

    # The closed form adds the leaves' images through A separately, which equals
    # A(sum) only when no carry crosses between them in A's mixed radix.  That holds
    # when A is one (unbounded, hence linear) leaf, or when B's non-trivial leaves,
    # sorted by stride, cover disjoint ranges: s_j * n_j <= s_{j+1}.
    if len(a_leaves) > 1:
        nontriv = sorted((d, n) for n, d in flatten(B) if n > 1 and d > 0)
        for (d0, n0), (d1, _) in zip(nontriv, nontriv[1:]):
            if d0 * n0 > d1:
                raise NotRepresentable("leaves of the right operand overlap")

    def leaf(n, s):
        parts = _compose_leaf(a_leaves, n, s)
        if len(parts) == 1:
            return parts[0]
        return tuple(p[0] for p in parts), tuple(p[1] for p in parts)

    shp, strd = _map_shape(B.shape, B.stride, leaf)
    return Layout(shp, strd, A.swz)


def compose_table(A: Layout, B: Layout) -> np.ndarray:
    """The function c -> A(B(c)) tabulated over B's 1-D index, evaluated directly
    (A coalesced, its last leaf unbounded).  Used to check ``compose``."""
    b = eval_indices(B, np.arange(size(B), dtype=np.int64))
    a_leaves = _coalesce_leaves(flatten(A)) or [(1, 0)]
    off = np.zeros_like(b)
    k = b.copy()
    for j, (n, d) in enumerate(a_leaves):
        if j == len(a_leaves) - 1:
            off += k * d
        else:
            off += (k % n) * d
            k //= n
    return swizzle(off, A.swz)


# ----------------------------------------------------------------------------
# Right inverse.  [CuTe algebra page, section 2.3]: the inverse layout answers
# which logical coordinate sits at a given offset.
# ----------------------------------------------------------------------------
def right_inverse(L: Layout) -> Layout:
    """Unswizzled L only.  Greedy chain from stride 1: pick the leaf whose stride
    equals the running product, append (extent : its colex weight in L)."""
    if L.swz is not None:
        raise NotRepresentable("swizzled layout: use right_inverse_fn")
    leaves = flatten(L)
    weights = []
    w = 1
    for n, _ in leaves:
        weights.append(w)
        w *= n
    cand = [(n, d, wt) for (n, d), wt in zip(leaves, weights) if n > 1 and d != 0]
    out = []
    expect = 1
    used = set()
    while True:
        hit = None
        for idx, (n, d, wt) in enumerate(cand):
            if idx not in used and d == expect:
                hit = idx
                break
        if hit is None:
            break
        used.add(hit)
        n, d, wt = cand[hit]
        out.append((n, wt))
        expect *= n
    return _from_leaves(out)


def right_inverse_fn(L: Layout):
    """Right inverse as a function: for a swizzled layout it is the unswizzled
    inverse applied after the swizzle (the swizzle is an involution).  Returns
    ``(f, m, dom)``: ``f(i)`` is defined for every ``i`` with ``dom(i)`` true, which
    are the ``i`` whose unswizzled offset is below ``m`` = size of the unswizzled
    inverse; ``dom`` holds for every ``i < m`` when there is no swizzle."""
    base = right_inverse(Layout(L.shape, L.stride))
    m = size(base)

    def pre(i):
        return swizzle(i, L.swz) if L.swz else i

    def f(i):
        return eval_index(base, pre(i))

    def dom(i):
        return 0 <= pre(i) < m

    return f, m, dom


# ----------------------------------------------------------------------------
# zipped_divide.  [CuTe algebra page, section 3.2]: split each mode by a tiler,
# giving ((tile modes), (rest modes)).
# ----------------------------------------------------------------------------
def zipped_divide(L: Layout, tiler: Sequence[int]) -> Layout:
    modes = top_modes(L)
    if len(tiler) > len(modes):
        raise ValueError("tiler has more entries than the layout has modes")
    tiles_s, tiles_d, rest_s, rest_d = [], [], [], []
    for j, m in enumerate(modes):
        n = size(m)
        t = tiler[j] if j < len(tiler) else 1
        if t < 1 or n % t:
            raise NotRepresentable(f"tile {t} does not divide extent {n}")
        tile = compose(m, Layout(t, 1))
        rest = compose(m, Layout(n // t, t))
        tiles_s.append(tile.shape)
        tiles_d.append(tile.stride)
        rest_s.append(rest.shape)
        rest_d.append(rest.stride)
    return Layout((tuple(tiles_s), tuple(rest_s)), (tuple(tiles_d), tuple(rest_d)), L.swz)


def slice_layout(L: Layout, coord):
    """[CuTe algebra page, section 3.2]: tile (3,5) of a zipped_divide is the layout
    with its rest mode fixed at (3,5) and its tile mode left free ("_").  ``coord``
    is congruent with (a prefix of the nesting of) L's shape: ``None`` keeps that
    sub-mode, an integer fixes it (split colexicographically inside the sub-mode, as
    in eval_coord).  Returns (layout of the kept sub-modes, offset of the fixed
    ones) with L(c) = offset + result(kept part of c).  The kept sub-modes are
    grouped by the top-level mode they belong to; when only one group is left, its
    leaves are the result's top-level modes.  A swizzle stays on the result
    when the offset is a multiple of 2^(M+S+B) -- the swizzle only reads and writes
    bits below that, so it then acts on the kept part alone; otherwise the slice is
    not a layout plus an offset."""
    def rec(c, shape, stride):
        if c is None:
            return [(shape, stride)], 0
        if isinstance(c, int):
            return [], _crd2off(c, shape, stride)
        if isinstance(shape, int) or len(c) != len(shape):
            raise ValueError("coordinate not congruent with shape")
        kept, off = [], 0
        for ci, si, di in zip(c, shape, stride):
            k, o = rec(ci, si, di)
            kept += k
            off += o
        return kept, off

    top = top_modes(L)
    if isinstance(L.shape, int) and not (isinstance(coord, tuple) and len(coord) == 1):
        coord = (coord,)  # a rank-1 layout: its one coordinate, bare or in a 1-tuple
    if len(coord) != len(top):
        raise ValueError("one coordinate per top-level mode")
    shapes, strides, off = [], [], 0
    for c, m in zip(coord, top):
        kept, o = rec(c, m.shape, m.stride)
        off += o
        if kept:
            shapes.append(kept[0][0] if len(kept) == 1 else tuple(k[0] for k in kept))
            strides.append(kept[0][1] if len(kept) == 1 else tuple(k[1] for k in kept))
    if not shapes:
        shapes, strides = [1], [0]
    elif len(shapes) == 1 and not isinstance(shapes[0], int):
        # one mode survives: its leaves are the result's modes (tile (3,5) is a 4 x 8
        # layout of its own)
        shapes, strides = list(_leaves(shapes[0])), list(_leaves(strides[0]))
    if L.swz is not None:
        b, m, s = L.swz
        if off % (1 << (m + s + b)):
            raise NotRepresentable("the fixed offset moves bits the swizzle reads")
    shp = shapes[0] if len(shapes) == 1 else tuple(shapes)
    std = strides[0] if len(strides) == 1 else tuple(strides)
    return Layout(shp, std, L.swz), off


# ----------------------------------------------------------------------------
# Complement, logical divide and products.  [CuTe algebra page, section 3.2]:
# dividing a layout into tiles and what is left over; [section 4.1]: a tile
# repeated over a grid with blocked_product (a 4x8 block over a 2x5 grid gives
# the "4x2, 8x5" layout).
# ----------------------------------------------------------------------------
def complement(A: Layout, M: int) -> Layout:
    """The layout of the positions A leaves out, up to size M: with A's leaves
    (n_i : d_i) of extent > 1 and stride > 0 sorted by stride, each d_{i+1} must be
    a multiple of n_i*d_i; the result is (d_0 : 1), (d_{i+1} / (n_i d_i) : n_i d_i)...,
    (ceil(M / (n_k d_k)) : n_k d_k), extent-1 leaves dropped, coalesced.  Then the
    concatenation (A, complement) is a bijection onto [0, multiple of n_k d_k >= M)."""
    if A.swz is not None:
        raise NotRepresentable("swizzled layout")
    leaves = sorted(((d, n) for n, d in flatten(A) if n > 1 and d > 0))
    out = []
    cur = 1  # stride reached so far (product n_i d_i of the last leaf)
    for d, n in leaves:
        if d % cur:
            raise NotRepresentable("strides are not nested")
        out.append((d // cur, cur))
        cur = n * d
    out.append((-(-M // cur), cur))
    return _from_leaves(_coalesce_leaves(out))


def _concat(A: Layout, B: Layout) -> Layout:
    return Layout((A.shape, B.shape), (A.stride, B.stride))


def logical_divide(A: Layout, B: Layout) -> Layout:
    """A o (B, complement(B, size(A))): mode 0 is the tile B picks out of A, mode 1
    enumerates the tiles."""
    return compose(A, _concat(B, complement(B, size(A))))


def logical_product(A: Layout, B: Layout) -> Layout:
    """(A, complement(A, size(A) * cosize(B)) o B): A repeated as B says."""
    C = complement(A, size(A) * cosize(B))
    return _concat(A, compose(C, B))


def blocked_product(A: Layout, B: Layout) -> Layout:
    """logical_product regrouped mode by mode: top-level mode i of the result is
    (mode i of A, mode i of the repeated B).  A and B need the same number of
    top-level modes."""
    ma, mb = top_modes(A), top_modes(B)
    if len(ma) != len(mb):
        raise ValueError("blocked_product needs layouts with the same number of modes")
    rep = logical_product(A, B)
    reps = top_modes(Layout(rep.shape[1], rep.stride[1]))
    if len(mb) == 1:
        reps = [Layout(rep.shape[1], rep.stride[1])]
    return Layout(tuple((x.shape, y.shape) for x, y in zip(ma, reps)),
                  tuple((x.stride, y.stride) for x, y in zip(ma, reps)))


# ----------------------------------------------------------------------------
# Injectivity.  [CuTe algebra page, section 2.3]: the inverse layout answers which
# logical coordinate a given offset holds, which is only one coordinate when no two
# coordinates share an offset.  The pages give no test; this is the definition
# (brute force) plus a sufficient condition on the strides.
# ----------------------------------------------------------------------------
BRUTE_INJECTIVE_LIMIT = 1 << 20


def is_injective_bruteforce(L: Layout) -> bool:
    offs = eval_indices(L, np.arange(size(L), dtype=np.int64))
    return len(np.unique(offs)) == len(offs)


def injective_sufficient(L: Layout) -> bool:
    """Sorted by stride, every stride exceeds the largest offset reachable by the
    smaller-stride leaves.  A stride-0 leaf of extent > 1 fails.  The swizzle is a
    bijection and does not matter."""
    leaves = sorted((d, n) for n, d in flatten(L) if n > 1)
    reach = 0
    for d, n in leaves:
        if d == 0 or d < reach + 1:
            return False
        reach += (n - 1) * d
    return True


# Limit of the exact check on the leaves that are not separated by stride: their
# combined extent.  Beyond it: "not proven injective".
EXACT_INJECTIVE_ELEMS = 1 << 22


def is_injective(L: Layout) -> bool:
    """Exact by brute force up to 2**20 elements.  Above that: with the leaves of
    extent > 1 sorted by stride, a leaf whose stride exceeds the largest offset
    reachable by the smaller ones is separated -- its translates of their image
    lie in disjoint ranges -- so L is injective iff the leaves up to the last one
    that is not separated are; those are brute-forced (within the limit above,
    else not proven).  A stride-0 leaf of extent > 1 is never injective."""
    if size(L) <= BRUTE_INJECTIVE_LIMIT:
        return is_injective_bruteforce(L)
    leaves = sorted((d, n) for n, d in flatten(L) if n > 1)
    if any(d == 0 for d, _ in leaves):
        return False
    last, reach = -1, 0
    for k, (d, n) in enumerate(leaves):
        if d <= reach:
            last = k
        reach += (n - 1) * d
    if last < 0:
        return True
    prefix = leaves[: last + 1]
    if math.prod(n for _, n in prefix) > EXACT_INJECTIVE_ELEMS:
        return False
    P = Layout(tuple(n for _, n in prefix), tuple(d for d, _ in prefix)) if len(prefix) > 1 else \
        Layout(prefix[0][1], prefix[0][0])
    return is_injective_bruteforce(P)


# ----------------------------------------------------------------------------
# Widest common vector.  [CuTe algebra page, section 2.3]: the largest k such that
# the inverses of both layouts agree on the first k offsets gives the widest copy
# unit.  The printed formula is garbled; the reading used: the largest power of two
# w with w*elem_bytes <= 16 such that the destination image is a union of aligned
# w-runs and, on each run, the source offsets are one aligned contiguous w-run in
# the same order.
# ----------------------------------------------------------------------------
def max_common_vector(Ls: Layout, Ld: Layout, elem_bytes: int) -> int:
    n = size(Ls)
    if size(Ld) != n:
        raise ValueError("size mismatch")
    ks = np.arange(n, dtype=np.int64)
    so = eval_indices(Ls, ks)
    do = eval_indices(Ld, ks)
    if len(np.unique(do)) != n:
        return 1
    order = np.argsort(do, kind="stable")
    do_s, so_s = do[order], so[order]
    w = 1
    best = 1
    while (2 * w) * elem_bytes <= 16:
        w *= 2
        if n % w:
            break
        blk_d = do_s.reshape(-1, w)
        blk_s = so_s.reshape(-1, w)
        u = np.arange(w, dtype=np.int64)
        ok = (
            np.all(blk_d[:, 0] % w == 0)
            and np.all(blk_d == blk_d[:, :1] + u)
            and np.all(blk_s[:, 0] % w == 0)
            and np.all(blk_s == blk_s[:, :1] + u)
        )
        if not ok:
            break
        best = w
    return best


# ----------------------------------------------------------------------------
# Joint flat form of a pair of layouts over one index space (unswizzled parts).
# [CuTe algebra page, section 2.3]: the copy between two layouts is planned from
# what the two have in common; the pages do not spell out how, and this is the
# common refinement of both leaf lists.
# Both leaf lists are split at the union of their prefix products, which must form
# a divisibility chain; extent-1 modes are dropped and neighbours contiguous on both
# sides merged.  With ``sort_by_dst`` the modes are sorted by (dst stride, src
# stride) and merged again until nothing changes.  Returns a list of
# (extent, src_stride, dst_stride) or None when no common refinement exists.
# ----------------------------------------------------------------------------
def joint_flat(Ls: Layout, Ld: Layout, sort_by_dst: bool = False):
    a = [(n, d) for n, d in flatten(Ls) if n > 1]
    b = [(n, d) for n, d in flatten(Ld) if n > 1]
    na = 1
    for n, _ in a:
        na *= n
    nb = 1
    for n, _ in b:
        nb *= n
    if na != nb:
        raise ValueError("size mismatch")

    def prefixes(lv):
        p, out = 1, [1]
        for n, _ in lv:
            p *= n
            out.append(p)
        return out

    cuts = sorted(set(prefixes(a)) | set(prefixes(b)))
    for x, y in zip(cuts, cuts[1:]):
        if y % x:
            return None

    def stride_at(lv, pos):
        p = 1
        for n, d in lv:
            if p <= pos < p * n:
                return d * (pos // p)
            p *= n
        raise AssertionError

    modes = []
    for x, y in zip(cuts, cuts[1:]):
        modes.append((y // x, stride_at(a, x), stride_at(b, x)))

    def merge(ms):
        out = []
        for e, s, d in ms:
            if e == 1:
                continue
            if out and s == out[-1][0] * out[-1][1] and d == out[-1][0] * out[-1][2]:
                out[-1] = (out[-1][0] * e, out[-1][1], out[-1][2])
            else:
                out.append((e, s, d))
        return out

    modes = merge(modes)
    if sort_by_dst:
        while True:
            nxt = merge(sorted(modes, key=lambda t: (t[2], t[1])))
            if nxt == modes:
                break
            modes = nxt
    return modes


# ----------------------------------------------------------------------------
# Thread maps.  [ThreadMap page, section 1.2]: row = tid / Pitch, col = tid % Pitch,
# offset = col + row * kRow.  [ThreadMap page, section 2.2]: the strip-mined map
# adds the strip within a group of Strips rows and a jump of Pitch*Strips*kRow per
# group.  The page's claim that Strips = 1 reduces to the base map does not hold
# under its own formula (the group jump becomes Pitch*kRow); both are kept as given.
# ----------------------------------------------------------------------------
def pitch_linear_offset(tid: int, pitch: int, krow: int) -> int:
    row, col = tid // pitch, tid % pitch
    return col + row * krow


def stripmined_offset(tid: int, pitch: int, strips: int, krow: int) -> int:
    q, r = tid // pitch, tid % pitch
    strip_id = q % strips
    group = q // strips
    return r + strip_id * krow + group * (pitch * strips * krow)


def stripmined_layout(pitch: int, strips: int, krow: int, threads: int) -> Layout:
    groups = -(-threads // (pitch * strips))
    return Layout((pitch, strips, groups), (1, krow, pitch * strips * krow))


def pitch_linear_layout(pitch: int, krow: int, threads: int) -> Layout:
    rows = -(-threads // pitch)
    return Layout((pitch, rows), (1, krow))


# ----------------------------------------------------------------------------
# The layout-remapping copy: for every index k in increasing order,
# dst[Ld(k)] = src[Ls(k)], elem_bytes opaque bytes each.  Positions of dst outside
# the image of Ld keep their bytes.  [CuTe algebra page, section 5.1]: a copy is
# made from a pair of layouts; [section 2.3]: the source and target differ only in
# layout.
# ----------------------------------------------------------------------------
def _view(buf: np.ndarray, eb: int) -> np.ndarray:
    if buf.dtype != np.uint8 or buf.ndim != 1:
        raise TypeError("byte buffers are flat uint8 arrays")
    if buf.nbytes % eb:
        raise ValueError("buffer length is not a multiple of elem_bytes")
    return buf.view(np.dtype((np.void, eb)))


def copy(src: np.ndarray, Ls: Layout, dst: np.ndarray, Ld: Layout, elem_bytes: int,
         ordered_alias: bool = False, chunk: int = 1 << 22) -> np.ndarray:
    """Returns a new dst byte buffer.  Raises if Ld is not injective and
    ``ordered_alias`` is False (the caller has not asked for the sequential rule)."""
    n = size(Ls)
    if size(Ld) != n:
        raise ValueError("size mismatch")
    sv = _view(src, elem_bytes)
    out = dst.copy()
    dv = _view(out, elem_bytes)
    if n == 0:
        return out
    if cosize(Ls) > len(sv) or cosize(Ld) > len(dv):
        raise IndexError("layout reaches beyond the buffer")
    if not is_injective(Ld):
        if not ordered_alias:
            raise ValueError("destination layout is not injective")
        if n > (1 << 20):
            raise ValueError("aliased oracle copy is limited to 2**20 elements")
        ks = np.arange(n, dtype=np.int64)
        so = eval_indices(Ls, ks)
        do = eval_indices(Ld, ks)
        for k in range(n):  # plain sequential loop: the last index wins
            dv[do[k]] = sv[so[k]]
        return out
    for k0 in range(0, n, chunk):
        ks = np.arange(k0, min(n, k0 + chunk), dtype=np.int64)
        dv[eval_indices(Ld, ks)] = sv[eval_indices(Ls, ks)]
    return out


def copy_sampled_check(src: np.ndarray, Ls: Layout, dst: np.ndarray, Ld: Layout,
                       elem_bytes: int, ks: np.ndarray) -> int:
    """For an injective Ld: count sampled indices k with dst[Ld(k)] != src[Ls(k)]."""
    sv = _view(src, elem_bytes)
    dv = _view(dst, elem_bytes)
    ks = np.asarray(ks, dtype=np.int64)
    a = sv[eval_indices(Ls, ks)]
    b = dv[eval_indices(Ld, ks)]
    return int(np.count_nonzero(a != b))
