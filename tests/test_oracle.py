"""The CPU oracle against what the pages and the mathematics fix.

Pins: values printed on the pages (tests/golden/*.txt, each with its citation),
closed forms, invariants, special cases that reduce to a NumPy routine, and brute
force on tiny layouts.  The last block plants plausible mistakes in the oracle and
checks that a pin catches each.
"""

import ast
import math
import re
import os
import random

import numpy as np
import pytest

import oracle as O
from oracle import layout as OL
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    header, rows = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("layout:") or line.startswith("map:"):
                key, val = line.split(":", 1)
                header[key] = val.strip()
            else:
                rows.append(line)
    return header, rows


# ---------------------------------------------------------------------------
# Printed grids and coordinates
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["rowmajor_4x2.txt", "colmajor_4x2.txt"])
def test_golden_grids(name):
    h, rows = _golden(name)
    L = O.parse(h["layout"])
    want = [[int(x) for x in r.split()] for r in rows]
    assert O.layout_grid(L) == want


@pytest.mark.parametrize("name", ["blocked_natural.txt", "swizzle_8x8.txt",
                                  "interleave_4x2x2.txt", "rank3_modes.txt"])
def test_golden_coords(name):
    h, rows = _golden(name)
    L = O.parse(h["layout"])
    for r in rows:
        crd, off = r.rsplit(" ", 1)
        assert O.eval_coord(L, ast.literal_eval(crd)) == int(off), r


@pytest.mark.parametrize("name", ["threadmap_p8_s4_k16.txt", "threadmap_p8_s2_k16.txt"])
def test_golden_threadmaps(name):
    h, rows = _golden(name)
    kv = dict(x.split("=") for x in h["map"].split()[1:])
    p, s, k, t = (int(kv[x]) for x in ("pitch", "strips", "krow", "threads"))
    L = O.stripmined_layout(p, s, k, t)
    for r in rows:
        t0, t1, o0 = (int(x) for x in r.split())
        for tid in range(t0, t1 + 1):
            assert O.stripmined_offset(tid, p, s, k) == o0 + tid - t0
            assert O.eval_index(L, tid) == o0 + tid - t0


def test_threadmap_layout_equals_formula_everywhere():
    for p in (1, 2, 4, 8, 32):
        for s in (1, 2, 3, 4):
            for k in (p, 16, 17, 64):
                t = 4 * p * s
                L = O.stripmined_layout(p, s, k, t)
                for tid in range(t):
                    assert O.eval_index(L, tid) == O.stripmined_offset(tid, p, s, k)
                B = O.pitch_linear_layout(p, k, t)
                for tid in range(t):
                    assert O.eval_index(B, tid) == O.pitch_linear_offset(tid, p, k)


def test_strips1_is_not_the_base_map():
    # [ThreadMap page, section 2.2] claims Strips = 1 gives the base map; its own
    # formula gives a group jump of Pitch*kRow instead of kRow.
    assert O.stripmined_offset(8, 8, 1, 16) == 128
    assert O.pitch_linear_offset(8, 8, 16) == 16


def test_swizzle_closed_form_and_properties():
    # [print_layout page, section 4.3]: offset = row*8 + (col ^ row)
    L = O.parse("Sw<3,0,3> o (8,8):(8,1)")
    for r in range(8):
        for c in range(8):
            assert O.eval_coord(L, (r, c)) == r * 8 + (c ^ r)
    # colex index order of the same layout
    assert [O.eval_index(L, k) for k in range(10)] == [0, 9, 18, 27, 36, 45, 54, 63, 1, 8]
    # bijection and involution for S >= B
    for b, m, s in [(3, 0, 3), (3, 3, 3), (2, 1, 4), (1, 0, 1), (3, 4, 3)]:
        o = np.arange(1 << (b + m + s + 1), dtype=np.int64)
        y = O.swizzle(o, (b, m, s))
        assert sorted(y.tolist()) == o.tolist()
        assert np.array_equal(O.swizzle(y, (b, m, s)), o)


def test_rowmajor_colmajor_samples():
    # [print_layout page, section 2.1]: (0,0)->0 (0,1)->1 (1,0)->2 (3,1)->7
    L = O.parse("(4,2):(2,1)")
    assert [L(0, 0), L(0, 1), L(1, 0), L(3, 1)] == [0, 1, 2, 7]


def test_index_and_coordinate_agree_colex():
    L = O.parse("((4,2),(2,4)):((2,16),(1,8))")
    for k in range(64):
        r, c = k % 8, k // 8
        assert O.eval_index(L, k) == O.eval_coord(L, (r, c))
        assert O.eval_coord(L, ((r % 4, r // 4), (c % 2, c // 2))) == O.eval_index(L, k)


def test_parse_format_roundtrip():
    for t in ["(4,2):(2,1)", "((4,2),(2,4)):((2,16),(1,8))", "Sw<3,3,3> o ((128,32),(64,64)):((64,524288),(1,8192))",
              "8:1", "(((2,2),3),5):(((1,2),4),12)"]:
        assert O.fmt(O.parse(t)) == t
    assert O.fmt(O.parse("(4,2,2):(_8,_2,_1)")) == "(4,2,2):(8,2,1)"
    with pytest.raises(ValueError):
        O.parse("(4,2):(1)")
    with pytest.raises(ValueError):
        O.parse("Sw<3,0,2> o 8:1")  # S < B


# ---------------------------------------------------------------------------
# The thread-value layout and composition
# ---------------------------------------------------------------------------
TV = "((4,8),2):((16,1),8)"


def test_tv_layout_partitions_the_tile():
    # [CuTe algebra page, sections 1 and 3.1]: 32 threads x 2 values cover an 8x8 tile
    L = O.parse(TV)
    offs = [O.eval_index(L, k) for k in range(64)]
    assert sorted(offs) == list(range(64))
    assert offs[:8] == [0, 16, 32, 48, 1, 17, 33, 49]


def test_compose_with_compact_colmajor_is_identity():
    # [CuTe algebra page, section 3.1]: composing the column-major user layout with
    # the thread-value layout gives the hardware layout, i.e. the TV layout itself
    A = O.parse("(8,8):(1,8)")
    B = O.parse(TV)
    assert O.fmt(O.compose(A, B)) == TV


def test_compose_padded():
    # [CuTe algebra page, section 2.2]: (8,8):(1,9) o TV skips the padding
    A, B = O.parse("(8,8):(1,9)"), O.parse(TV)
    R = O.compose(A, B)
    assert O.fmt(R) == "((4,8),2):((18,1),9)"
    table = O.compose_table(A, B)
    assert np.array_equal(O.eval_indices(R, np.arange(64)), table)
    assert not np.any(table % 9 == 8)  # never lands on a pad word
    assert O.is_injective(R)


def _rand_layout(rng, max_leaves=4, max_ext=4, max_stride=16, swz_p=0.0, allow_zero=True):
    nl = rng.randint(1, max_leaves)
    ext = [rng.randint(1, max_ext) for _ in range(nl)]
    lo = 0 if allow_zero else 1
    st = [rng.randint(lo, max_stride) for _ in range(nl)]
    # random grouping into top-level modes
    modes, i = [], 0
    while i < nl:
        j = rng.randint(i + 1, nl)
        modes.append((tuple(ext[i:j]), tuple(st[i:j])))
        i = j
    shp = tuple(m[0] if len(m[0]) > 1 else m[0][0] for m in modes)
    sd = tuple(m[1] if len(m[1]) > 1 else m[1][0] for m in modes)
    if len(shp) == 1:
        shp, sd = shp[0], sd[0]
    swz = None
    if rng.random() < swz_p:
        b = rng.randint(1, 2)
        swz = (b, rng.randint(0, 2), rng.randint(b, 3))
    return O.Layout(shp, sd, swz)


def test_compose_closed_form_matches_table_random():
    rng = random.Random(1234)
    hits = 0
    for _ in range(3000):
        A = _rand_layout(rng, swz_p=0.2)
        B = _rand_layout(rng, max_stride=6)
        try:
            R = O.compose(A, B)
        except OL.NotRepresentable:
            continue
        hits += 1
        assert np.array_equal(O.eval_indices(R, np.arange(O.size(B))), O.compose_table(A, B)), (A, B)
    assert hits > 1000


def test_compose_associative_random():
    rng = random.Random(99)
    hits = 0
    for _ in range(3000):
        A = _rand_layout(rng)
        B = _rand_layout(rng, max_stride=4)
        C = _rand_layout(rng, max_stride=4)
        # associativity is a statement about functions inside their domains: the
        # unbounded extension of a last leaf is not part of it
        if O.cosize(C) > O.size(B) or O.cosize(B) > O.size(A):
            continue
        try:
            left = O.compose(O.compose(A, B), C)
            right = O.compose(A, O.compose(B, C))
        except OL.NotRepresentable:
            continue
        hits += 1
        n = np.arange(O.size(C))
        assert np.array_equal(O.eval_indices(left, n), O.eval_indices(right, n)), (A, B, C)
    assert hits > 200


def test_coalesce_preserves_function_and_is_canonical():
    rng = random.Random(7)
    assert O.fmt(O.coalesce(O.parse("(8,8):(1,8)"))) == "64:1"
    assert O.fmt(O.coalesce(O.parse("(1,4,1,2):(5,1,7,4)"))) == "8:1"
    for _ in range(3000):
        L = _rand_layout(rng, swz_p=0.3)
        C = O.coalesce(L)
        n = np.arange(O.size(L))
        assert np.array_equal(O.eval_indices(L, n), O.eval_indices(C, n))
        lv = O.flatten(C)
        if len(lv) > 1:
            assert all(e > 1 for e, _ in lv)
            assert all(lv[i + 1][1] != lv[i][0] * lv[i][1] for i in range(len(lv) - 1))


# ---------------------------------------------------------------------------
# Right inverse
# ---------------------------------------------------------------------------
def test_right_inverse_tv():
    R = O.right_inverse(O.parse(TV))
    assert O.fmt(R) == "(8,2,4):(4,32,1)"
    L = O.parse(TV)
    for k in range(64):
        assert O.eval_index(R, O.eval_index(L, k)) == k


def test_right_inverse_property_random():
    rng = random.Random(5)
    for _ in range(3000):
        L = _rand_layout(rng, swz_p=0.3)
        f, m, dom = O.right_inverse_fn(L)
        span = m if L.swz is None else 2 * m + (1 << sum(L.swz))
        checked = 0
        for i in range(span):
            if dom(i):
                assert O.eval_index(L, f(i)) == i, (L, i)
                checked += 1
        assert checked == m
        # bijective onto [0, size): the inverse is two-sided
        offs = O.eval_indices(L, np.arange(O.size(L)))
        if sorted(offs.tolist()) == list(range(O.size(L))):
            assert m == O.size(L)
            for k in range(O.size(L)):
                assert f(int(offs[k])) == k


# ---------------------------------------------------------------------------
# zipped_divide
# ---------------------------------------------------------------------------
def test_zipped_divide_tile_3_5():
    # [CuTe algebra page, section 3.2]: 128x128 column-major data split by a 4x8
    # tiler; block (3,5) read as the tile at rest coordinate (3,5)
    L = O.parse("(128,128):(1,128)")
    Z = O.zipped_divide(L, (4, 8))
    assert O.fmt(Z) == "((4,8),(32,16)):((1,128),(4,1024))"
    offs = sorted(O.eval_coord(Z, ((i, j), (3, 5))) for i in range(4) for j in range(8))
    want = sorted(r + 128 * c for r in range(12, 16) for c in range(40, 48))
    assert offs == want and offs[0] == 5132 and offs[-1] == 6031


def test_slice_tile_3_5_of_the_zipped_divide():
    # [CuTe algebra page, section 3.2]: the tile at rest coordinate (3,5), the tile
    # mode left free: a 4x8 layout whose offsets are the block {r + 128 c : r in
    # [12,16), c in [40,48)} of the column-major 128x128 data
    Z = O.zipped_divide(O.parse("(128,128):(1,128)"), (4, 8))
    T, off = O.slice_layout(Z, (None, (3, 5)))
    assert off == 3 * 4 + 5 * 1024 == 5132
    assert O.fmt(T) == "(4,8):(1,128)"
    got = sorted(off + O.eval_index(T, k) for k in range(32))
    assert got == sorted(r + 128 * c for r in range(12, 16) for c in range(40, 48))
    # the rest coordinate as one integer (colex inside the mode): 3 + 32 * 5
    assert O.slice_layout(Z, (None, 3 + 32 * 5)) == (T, off)
    # fixing the tile instead: the tile's element (1, 2) in every tile
    R, off2 = O.slice_layout(Z, ((1, 2), None))
    assert off2 == 1 + 2 * 128 and O.fmt(R) == "(32,16):(4,1024)"
    # everything fixed: a single offset; nothing fixed: the layout itself
    assert O.slice_layout(Z, ((3, 7), (31, 15))) == (O.Layout(1, 0), 3 + 7 * 128 + 31 * 4 + 15 * 1024)
    assert 3 + 7 * 128 + 31 * 4 + 15 * 1024 == 128 * 128 - 1  # the last element
    A, z = O.slice_layout(Z, (None, None))
    assert z == 0 and O.fmt(A) == O.fmt(Z)


def test_slice_definition_random():
    """L(c) == offset + slice(L, fixed)(free part of c), for every c whose fixed
    entries match, on random nested layouts; keeping leaves inside a nested mode."""
    rng = random.Random(5)
    hits = 0
    for _ in range(400):
        L = _rand_layout(rng, max_leaves=5)
        top = O.top_modes(L)
        # per top-level mode: None keeps it, an integer fixes it
        coord = tuple(None if rng.random() < 0.5 else rng.randrange(O.size(m)) for m in top)
        S, off = O.slice_layout(L, coord)
        free = [i for i, c in enumerate(coord) if c is None]
        sizes = [O.size(top[i]) for i in free]
        assert O.size(S) == math.prod(sizes)
        for k in range(O.size(S)):
            full, r = list(coord), k
            for i, n in zip(free, sizes):  # the kept modes, colex
                full[i], r = r % n, r // n
            c = tuple(full) if len(top) > 1 else full[0]
            assert O.eval_coord(L, c) == off + O.eval_index(S, k), (O.fmt(L), coord)
        hits += 1
    assert hits == 400
    # a leaf inside a nested mode: ((4,2),3):((1,8),4) keeping the 4, fixing the 2 at 1
    S, off = O.slice_layout(O.parse("((4,2),3):((1,8),4)"), ((None, 1), None))
    assert off == 8 and O.fmt(S) == "(4,3):(1,4)"


def test_slice_of_a_swizzled_layout():
    # the retile's destination: tile (r_t, c_t) of 128 x 64 elements starts at a
    # multiple of 8192, past every bit Sw<3,3,3> reads or writes (bits 3..8), so the
    # slice keeps the swizzle and the tile's own offsets are Sw(64 r + c)
    L = O.parse("Sw<3,3,3> o ((128,32),(64,64)):((64,524288),(1,8192))")
    S, off = O.slice_layout(L, ((None, 2), (None, 5)))
    assert off == 2 * 524288 + 5 * 8192 and S.swz == (3, 3, 3)
    for r in range(128):
        for c in range(64):
            assert O.eval_coord(L, ((r, 2), (c, 5))) == off + O.eval_coord(S, (r, c))
    # a base inside the swizzled bits is not a layout plus an offset
    with pytest.raises(OL.NotRepresentable):
        O.slice_layout(L, ((1, None), None))


def test_zipped_divide_definition_random():
    rng = random.Random(11)
    for _ in range(500):
        r, c = rng.choice([2, 4, 6, 8, 12]), rng.choice([2, 3, 4, 8])
        sr, sc = rng.randint(0, 5), rng.randint(1, 20)
        L = O.Layout((r, c), (sr, sc))
        tr = rng.choice([t for t in (1, 2, 3, 4) if r % t == 0])
        tc = rng.choice([t for t in (1, 2, 4) if c % t == 0])
        Z = O.zipped_divide(L, (tr, tc))
        for i in range(tr):
            for j in range(tc):
                for p in range(r // tr):
                    for q in range(c // tc):
                        assert O.eval_coord(Z, ((i, j), (p, q))) == O.eval_coord(L, (i + tr * p, j + tc * q))


# ---------------------------------------------------------------------------
# Injectivity
# ---------------------------------------------------------------------------
def test_blocked_layout_is_not_injective():
    L = O.parse("((4,2),(2,4)):((2,16),(1,8))")
    offs = O.eval_indices(L, np.arange(64))
    assert O.cosize(L) == 48 and len(set(offs.tolist())) == 48
    counts = np.bincount(offs, minlength=48)
    assert set(np.nonzero(counts == 2)[0].tolist()) == set(range(16, 32))
    assert not O.is_injective(L)


def test_rank3_with_holes_is_injective():
    L = O.parse("(4,2,2):(8,2,1)")
    offs = sorted(O.eval_indices(L, np.arange(16)).tolist())
    assert offs == [0, 1, 2, 3, 8, 9, 10, 11, 16, 17, 18, 19, 24, 25, 26, 27]
    assert O.is_injective(L)


def test_injective_sufficient_is_sound():
    rng = random.Random(3)
    for _ in range(5000):
        L = _rand_layout(rng, swz_p=0.3)
        if O.injective_sufficient(L):
            assert O.is_injective_bruteforce(L), L
    # a known injective layout the sufficient test cannot prove
    L = O.parse("(3,2):(2,3)")
    assert O.is_injective_bruteforce(L) and not O.injective_sufficient(L)


def test_injective_by_separated_leaves_equals_brute_force(monkeypatch):
    """The large-layout rule (separated leaves, brute force on the rest) used at
    every size by lowering the brute-force limit to 0, against the definition
    (every index to a distinct offset) on random layouts, including swizzled ones,
    stride-0 leaves and layouts the plain sufficient test cannot prove."""
    rng = random.Random(8)
    monkeypatch.setattr(OL, "BRUTE_INJECTIVE_LIMIT", 0)
    seen = {True: 0, False: 0}
    hard = 0
    for _ in range(6000):
        L = _rand_layout(rng, max_leaves=5, max_ext=5, max_stride=12, swz_p=0.2)
        want = O.is_injective_bruteforce(L)
        assert O.is_injective(L) == want, O.fmt(L)
        seen[want] += 1
        hard += want and not O.injective_sufficient(L)
    assert min(seen.values()) > 1000 and hard > 100, (seen, hard)
    monkeypatch.undo()
    # large: (3,2,M):(2,3,8) is injective for every M (the first two leaves give
    # {0,2,3,4,5,7} inside [0,8)); (3,2,M):(2,2,8) repeats 2; a stride-0 leaf repeats
    M = (1 << 22) + 3
    assert O.is_injective(O.parse(f"(3,2,{M}):(2,3,8)"))
    assert not O.is_injective(O.parse(f"(3,2,{M}):(2,2,8)"))
    assert not O.is_injective(O.parse(f"(2,{M}):(0,1)"))
    small = O.parse("(3,2,1000):(2,3,8)")
    assert O.is_injective_bruteforce(small)
    # beyond the limits of the exact part: not proven
    assert not O.is_injective(O.parse(f"({1 << 13},{1 << 12}):(1,{(1 << 13) - 1})"))


# ---------------------------------------------------------------------------
# Widest common vector
# ---------------------------------------------------------------------------
def _vector_copy(src, Ls, dst, Ld, eb, w):
    """Copy in w-element units: each aligned destination run takes w contiguous
    source elements starting at the source offset of its first element."""
    sv = src.view(np.dtype((np.void, eb)))
    out = dst.copy()
    dv = out.view(np.dtype((np.void, eb)))
    n = O.size(Ls)
    ks = np.arange(n)
    so, do = O.eval_indices(Ls, ks), O.eval_indices(Ld, ks)
    for k in range(n):
        if do[k] % w == 0:
            dv[do[k]:do[k] + w] = sv[so[k]:so[k] + w]
    return out


def test_common_vector_pins():
    assert O.max_common_vector(O.parse("64:1"), O.parse("64:1"), 2) == 8
    assert O.max_common_vector(O.parse("64:1"), O.parse("64:1"), 4) == 4
    assert O.max_common_vector(O.parse("(8,8):(8,1)"), O.parse("(8,8):(1,8)"), 2) == 1
    assert O.max_common_vector(O.parse("(4,4):(1,5)"), O.parse("(4,4):(1,4)"), 4) == 1
    assert O.max_common_vector(O.parse("(8,4):(1,10)"), O.parse("(8,4):(1,8)"), 2) == 2
    # aliased destination
    assert O.max_common_vector(O.parse("(8,8):(1,8)"), O.parse("((4,2),(2,4)):((2,16),(1,8))"), 4) == 1
    w = W.small("retile")
    assert O.max_common_vector(O.parse(w.src_layout), O.parse(w.dst_layout), 2) == 8


def test_common_vector_copy_equivalence_random():
    rng = random.Random(21)
    for _ in range(400):
        Ld = _rand_layout(rng, max_stride=12, swz_p=0.2, allow_zero=False)
        if not O.is_injective(Ld):
            continue
        # a source with the same size: a random permutation-like layout
        Ls = _rand_layout(rng, max_stride=12, allow_zero=False)
        if O.size(Ls) != O.size(Ld):
            Ls = O.Layout(O.size(Ld), rng.choice([1, 2]))
        eb = rng.choice([1, 2, 4])
        w = O.max_common_vector(Ls, Ld, eb)
        src = np.random.default_rng(0).integers(0, 256, (O.cosize(Ls) + 16) * eb, dtype=np.uint8)
        dst = np.full((O.cosize(Ld) + 16) * eb, 0xA5, dtype=np.uint8)
        ref = O.copy(src, Ls, dst, Ld, eb)
        assert np.array_equal(_vector_copy(src, Ls, dst, Ld, eb, w), ref), (Ls, Ld, w)


# ---------------------------------------------------------------------------
# Joint flat form
# ---------------------------------------------------------------------------
JOINT_FULL = {
    # per workload: (extent, src stride, dst stride) after sorting by dst stride
    "transpose": [(8192, 8192, 1), (8192, 1, 8192)],
    "retile": [(64, 1, 1), (128, 4096, 64), (64, 64, 8192), (32, 524288, 524288)],
    "interleave": [(2, 524288, 1), (524288, 1, 2), (256, 1048576, 1048576)],
    "interleave_cm": [(2, 524288, 1), (4096, 128, 2), (128, 1, 8192), (256, 1048576, 1048576)],
    "nhwc2nchw": [(3136, 256, 1), (256, 1, 3136), (128, 802816, 802816)],
    "padtiles": [(4, 18, 1), (8, 1, 4), (2, 9, 32), (1048576, 72, 64)],
    "tile8x8": [(8, 1, 1), (8, 8, 8)],  # dst (8,8) refinement, aliased: not used
    # block j's columns follow block j-1's in the destination: one rectangular transpose
    "shard_pack": [(1024, 8192, 1), (8192, 1, 1024)],
    "rgb_nhwc2nchw": [(50176, 3, 1), (3, 1, 50176), (512, 150528, 150528)],
}


@pytest.mark.parametrize("name", ["transpose", "retile", "interleave", "interleave_cm", "nhwc2nchw", "padtiles",
                                  "shard_pack", "rgb_nhwc2nchw"])
def test_joint_flat_of_workloads(name):
    w = W.full(name)
    got = O.joint_flat(O.parse(w.src_layout), O.parse(w.dst_layout), sort_by_dst=True)
    assert got == JOINT_FULL[name]


def test_joint_flat_random_function():
    rng = random.Random(8)
    hits = 0
    for _ in range(3000):
        Ls = _rand_layout(rng, swz_p=0.0)
        exts = [e for e, _ in O.flatten(Ls)]
        rng.shuffle(exts)
        Ld = O.Layout(tuple(exts), tuple(rng.randint(0, 9) for _ in exts)) if len(exts) > 1 else O.Layout(exts[0], 3)
        for sort in (False, True):
            jm = O.joint_flat(Ls, Ld, sort_by_dst=sort)
            if jm is None:
                continue
            hits += 1
            n = O.size(Ls)
            ks = np.arange(n)
            pairs = set(zip(O.eval_indices(Ls, ks).tolist(), O.eval_indices(Ld, ks).tolist()))
            # evaluate the joint modes over their own colex index
            s = np.zeros(n, np.int64)
            d = np.zeros(n, np.int64)
            k = ks.copy()
            for e, ss, dd in jm:
                s += (k % e) * ss
                d += (k % e) * dd
                k //= e
            assert set(zip(s.tolist(), d.tolist())) == pairs
            if not sort:  # unsorted: the same function of k
                assert np.array_equal(s, O.eval_indices(Ls, ks))
    assert hits > 1000
    assert O.joint_flat(O.parse("(6,4):(1,6)"), O.parse("(4,6):(1,4)")) is None


# ---------------------------------------------------------------------------
# Copies: special cases that reduce to NumPy routines, invariants, aliasing
# ---------------------------------------------------------------------------
def _run(w):
    src, dst = W.make_src(w), W.make_dst(w)
    out = O.copy(src, O.parse(w.src_layout), dst, O.parse(w.dst_layout), w.elem_bytes,
                 ordered_alias=w.ordered_alias)
    return src, out


def test_copy_transpose_is_numpy_transpose():
    w = W.small("transpose")
    n = 520
    src, out = _run(w)
    s = src.view(np.uint16).reshape(n, n)
    assert np.array_equal(out.view(np.uint16).reshape(n, n), s.T)


def test_copy_retile_is_reshape_plus_chunk_xor():
    w = W.small("retile")
    n = 512
    src, out = _run(w)
    s = src.view(np.uint16).reshape(n // 128, 128, n // 64, 64).transpose(0, 2, 1, 3)  # tiles row-major
    tiles = s.reshape(-1, 128, 8, 8)                       # (tile, row, chunk, elem)
    rows = np.arange(128)[:, None]
    chunks = np.arange(8)[None, :]
    placed = np.empty_like(tiles)
    placed[:, rows, chunks ^ (rows % 8)] = tiles[:, rows, chunks]
    assert np.array_equal(out.view(np.uint16), placed.reshape(-1))


def test_retile_samples_full_size():
    L = O.parse(W.full("retile").dst_layout)
    samples = {(0, 0): 0, (1, 0): 72, (1, 8): 64, (0, 64): 8192, (128, 0): 524288, (4095, 4095): 16777159}
    for (r, c), off in samples.items():
        assert O.eval_coord(L, (r, c)) == off
        # closed form: tile-major base plus the swizzled in-tile offset
        t = 8192 * (64 * (r // 128) + c // 64)
        assert t + O.swizzle(64 * (r % 128) + c % 64, (3, 3, 3)) == off


def test_copy_interleave_is_numpy_transpose():
    w = W.small("interleave")
    b, h, s, d = 2, 4, 72, 128
    src, out = _run(w)
    x = src.view(np.uint16).reshape(b, h // 2, 2, s, d).transpose(0, 1, 3, 4, 2)
    assert np.array_equal(out.view(np.uint16), x.reshape(-1))
    L = O.parse(W.full("interleave").dst_layout)
    assert L(0, 1, 0, 0) == 1 and L(0, 0, 0, 1) == 2 and L(0, 2, 0, 0) == 1048576


def test_copy_nhwc2nchw_is_numpy_transpose():
    w = W.small("nhwc2nchw")
    src, out = _run(w)
    x = src.view(np.uint16).reshape(3, 7, 9, 40).transpose(0, 3, 1, 2)
    assert np.array_equal(out.view(np.uint16), x.reshape(-1))


def test_copy_padtiles_is_take():
    w = W.small("padtiles")
    src, out = _run(w)
    table = np.array([18 * (k % 4) + (k // 4) % 8 + 9 * (k // 32) for k in range(64)])
    assert table[:8].tolist() == [0, 18, 36, 54, 1, 19, 37, 55] and table[-1] == 70
    s = src.view(np.uint32).reshape(-1, 72)
    assert np.array_equal(out.view(np.uint32).reshape(-1, 64), np.take(s, table, axis=1))
    # the destination layout is compact and the source read never touches a pad word
    assert not np.any(table % 9 == 8)


def test_copy_tile8x8_aliased_last_writer():
    w = W.tile8x8()
    src = W.make_src(w)
    with pytest.raises(ValueError):
        O.copy(src, O.parse(w.src_layout), W.make_dst(w), O.parse(w.dst_layout), 4)
    out = O.copy(src, O.parse(w.src_layout), W.make_dst(w), O.parse(w.dst_layout), 4, ordered_alias=True)
    want_idx = [0, 8, 1, 9, 2, 10, 3, 11, 16, 24, 17, 25, 18, 26, 19, 27, 32, 40, 33, 41, 34, 42, 35, 43,
                48, 56, 49, 57, 50, 58, 51, 59, 36, 44, 37, 45, 38, 46, 39, 47, 52, 60, 53, 61, 54, 62, 55, 63]
    sv, ov = src.view(np.uint32), out.view(np.uint32)
    assert ov[:48].tolist() == sv[want_idx].tolist()
    assert np.all(out.reshape(64, 4)[48:] == 0xA5)
    # a first-writer (or print-order) rule would differ at 16..31
    first = [4, 12, 5, 13, 6, 14, 7, 15, 20, 28, 21, 29, 22, 30, 23, 31]
    assert ov[16:32].tolist() != sv[first].tolist()


def test_copy_holes_keep_sentinel_and_permutation():
    rng = np.random.default_rng(4)
    Ls, Ld = O.parse("16:1"), O.parse("(4,2,2):(8,2,1)")
    src = rng.integers(0, 256, 16 * 2, dtype=np.uint8)
    out = O.copy(src, Ls, np.full(28 * 2, 0xA5, np.uint8), Ld, 2)
    ov = out.view(np.uint16)
    image = set(O.eval_indices(Ld, np.arange(16)).tolist())
    for o in range(28):
        if o not in image:
            assert ov[o] == 0xA5A5
    assert sorted(ov[sorted(image)].tolist()) == sorted(src.view(np.uint16).tolist())


def test_copy_sampled_check_counts_planted_mismatches():
    # The sampled checker against a destination built by NumPy's transpose, not by
    # the oracle: index k of (48,48):(48,1) -> (48,48):(1,48) is (i, j) = (k % 48,
    # k // 48) colex, read at 48 i + j and written at i + 48 j.
    n = 48
    rng = np.random.default_rng(11)
    src = rng.integers(0, 1 << 16, n * n, dtype=np.uint16)
    good = np.full(n * n + 16, 0xA5A5, np.uint16)  # 16 words past the image: holes
    good[: n * n] = src.reshape(n, n).T.reshape(-1)
    Ls, Ld = O.parse("(48,48):(48,1)"), O.parse("(48,48):(1,48)")
    ks = rng.choice(n * n, 300, replace=False)

    def check(dst):
        return O.copy_sampled_check(src.view(np.uint8), Ls, dst.view(np.uint8), Ld, 2, ks)

    assert check(good) == 0
    holes = good.copy()
    holes[n * n:] = 0x1234  # bytes outside the image are not the checker's business
    assert check(holes) == 0
    bad = good.copy()
    planted = ks[[0, 5, 17, 99, 150, 222, 299]]
    for k in planted:
        bad[(k % n) + n * (k // n)] ^= 0x0100  # one flipped bit at a sampled destination
    assert check(bad) == len(planted)
    # a wrong element at an index outside the sample is not counted
    outside = np.setdiff1d(np.arange(n * n), ks)[:5]
    for k in outside:
        bad[(k % n) + n * (k // n)] ^= 0x0001
    assert check(bad) == len(planted)
    # every sampled index wrong: the count is the sample size
    assert check(np.zeros_like(good)) == int(np.count_nonzero(src[(ks % n) * n + ks // n] != 0))
    # a swizzled destination: the checker must apply the swizzle (Sw<3,0,3> on an 8x8
    # row-major tile puts (r, c) at 8 r + (c ^ r), [print_layout page, section 4.3])
    s8 = rng.integers(0, 1 << 32, 64, dtype=np.uint32)
    d8 = np.empty(64, np.uint32)
    for r in range(8):
        for c in range(8):
            d8[8 * r + (c ^ r)] = s8[8 * r + c]
    Lrow, Lsw = O.parse("(8,8):(8,1)"), O.parse("Sw<3,0,3> o (8,8):(8,1)")
    all64 = np.arange(64)
    assert O.copy_sampled_check(s8.view(np.uint8), Lrow, d8.view(np.uint8), Lsw, 4, all64) == 0
    # the unswizzled destination differs wherever c ^ r != c, i.e. in every row but 0
    assert O.copy_sampled_check(s8.view(np.uint8), Lrow, s8.view(np.uint8), Lsw, 4, all64) == 56


def test_copy_bits_survive():
    # NaN payloads, infinities, subnormals: bytes move unchanged
    src = np.array([0x7E01, 0xFC00, 0x0001, 0x8000, 0x7FFF, 0xFFFF], np.uint16).view(np.uint8)
    out = O.copy(src, O.parse("6:1"), np.zeros(12, np.uint8), O.parse("(2,3):(3,1)"), 2)
    assert out.view(np.uint16).tolist() == [0x7E01, 0x0001, 0x7FFF, 0xFC00, 0x8000, 0xFFFF]


def test_copy_elem16_and_elem8():
    rng = np.random.default_rng(9)
    for eb in (8, 16):
        src = rng.integers(0, 256, 12 * eb, dtype=np.uint8)
        out = O.copy(src, O.parse("(3,4):(4,1)"), np.zeros(12 * eb, np.uint8), O.parse("(3,4):(1,3)"), eb)
        s = src.reshape(3, 4, eb)  # element (i,j) at src 4i+j ... dst i+3j
        o = out.reshape(4, 3, eb)
        for i in range(3):
            for j in range(4):
                assert np.array_equal(o[j, i], s[i, j])


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by a pin above
# ---------------------------------------------------------------------------
def _lex_eval(L, k):  # plausible mistake: last leaf fastest
    off = 0
    for n, d in reversed(O.flatten(L)):
        off += (k % n) * d
        k //= n
    return off


def test_planted_lexicographic_order_is_caught():
    h, rows = _golden("threadmap_p8_s4_k16.txt")
    L = O.stripmined_layout(8, 4, 16, 64)
    assert [_lex_eval(L, t) for t in range(8)] != list(range(8))


def test_planted_swizzle_direction_is_caught(monkeypatch):
    def wrong(o, swz):  # XORs the low bits into the high bits instead
        if swz is None:
            return o
        b, m, s = swz
        return o ^ ((o << s) & ((((1 << b) - 1) << m) << s))

    monkeypatch.setattr(OL, "swizzle", wrong)
    L = O.parse("Sw<3,0,3> o (8,8):(8,1)")
    assert O.eval_coord(L, (2, 0)) != 18


def test_planted_compose_transposed_operands_is_caught():
    A, B = O.parse("(8,8):(1,9)"), O.parse(TV)
    try:
        wrong = O.fmt(O.compose(B, A))
    except OL.NotRepresentable:
        wrong = None
    assert wrong != "((4,8),2):((18,1),9)"


def test_planted_dropped_alignment_in_vector_width_is_caught():
    # The source run for each 4-wide destination run of this pitched copy is
    # contiguous but starts at 5, 10, 15: a 16-byte load there is misaligned.  A
    # width rule that forgot the source alignment would answer 4; the pin says 1.
    Ls, Ld = O.parse("(4,4):(1,5)"), O.parse("(4,4):(1,4)")
    so = O.eval_indices(Ls, np.arange(16)).reshape(4, 4)
    assert np.all(so == so[:, :1] + np.arange(4))          # contiguous runs ...
    assert not np.all(so[:, 0] % 4 == 0)                   # ... not aligned
    assert O.max_common_vector(Ls, Ld, 4) == 1


# ---------------------------------------------------------------------------
# NumPy closed forms used for whole-buffer checks at full size: each equals the
# oracle's copy at a reduced size with the same structure
# ---------------------------------------------------------------------------
def test_forms_equal_oracle_copy():
    from oracle import forms as F

    cases = {
        "transpose": lambda s: F.transpose(s, 520),
        "retile": lambda s: F.retile(s, 512),
        "interleave": lambda s: F.interleave(s, 2, 4, 72, 128),
        "interleave_cm": lambda s: F.interleave_cm(s, 2, 4, 72, 136),
        "nhwc2nchw": lambda s: F.nhwc2nchw(s, 3, 7, 9, 40),
        "padtiles": lambda s: F.padtiles(s, 1000),
        "shard_pack": lambda s: F.shard_pack(s, 520, 2112, 8),
        "rgb_nhwc2nchw": lambda s: F.nhwc2nchw(s, 3, 17, 40, 3),
        "head_split": lambda s: F.head_split(s, 2, 70, 6, 128),
    }
    for name, form in cases.items():
        w = W.small(name)
        src, out = _run(w)
        assert np.array_equal(form(src), out), name
    # the channel shuffles at other element sizes, both directions
    rng = np.random.default_rng(12)
    for eb in (1, 4, 8):
        n, h, wd, c = 2, 5, 6, 3
        hw = h * wd
        nhwc = O.parse(f"({n},{h},{wd},{c}):({hw * c},{wd * c},{c},1)")
        nchw = O.parse(f"({n},{h},{wd},{c}):({hw * c},{wd},1,{hw})")
        src = rng.integers(0, 256, n * hw * c * eb, dtype=np.uint8)
        blank = np.zeros_like(src)
        assert np.array_equal(F.nhwc2nchw(src, n, h, wd, c, eb), O.copy(src, nhwc, blank, nchw, eb)), eb
        assert np.array_equal(F.nchw2nhwc(src, n, h, wd, c, eb), O.copy(src, nchw, blank, nhwc, eb)), eb
    # batched transposes of 1- to 16-byte elements, square and not, one matrix or several
    for eb, (m, r, c) in [(1, (1, 5, 7)), (2, (3, 4, 6)), (4, (2, 7, 3)), (8, (1, 6, 6)), (16, (2, 3, 5))]:
        src = rng.integers(0, 256, m * r * c * eb, dtype=np.uint8)
        Ls = O.parse(f"({r},{c},{m}):({c},1,{r * c})")
        Ld = O.parse(f"({r},{c},{m}):(1,{r},{r * c})")
        assert np.array_equal(F.transpose_batched(src, m, r, c, eb), O.copy(src, Ls, np.zeros_like(src), Ld, eb)), eb
    # strided copies between flat layouts: permutes with padding, a gather of every second row,
    # a reversal of modes and a broadcast-free injective scatter, against the oracle's copy
    for eb, shape, ss, sd in [(2, (4, 3, 5), (1, 4, 12), (15, 5, 1)), (4, (6, 7), (1, 8), (7, 1)),
                              (1, (3, 4, 2), (1, 6, 3), (1, 3, 12)), (8, (5, 4), (1, 10), (1, 5)),
                              (16, (2, 3, 4), (12, 4, 1), (1, 2, 6))]:
        ns = 1 + sum((e - 1) * x for e, x in zip(shape, ss))
        nd = 1 + sum((e - 1) * x for e, x in zip(shape, sd))
        src = rng.integers(0, 256, ns * eb, dtype=np.uint8)
        dst = rng.integers(0, 256, nd * eb, dtype=np.uint8)
        Ls = O.parse("(" + ",".join(map(str, shape)) + "):(" + ",".join(map(str, ss)) + ")")
        Ld = O.parse("(" + ",".join(map(str, shape)) + "):(" + ",".join(map(str, sd)) + ")")
        assert np.array_equal(F.strided_copy(src, shape, ss, dst, sd, eb), O.copy(src, Ls, dst, Ld, eb)), (eb, shape)
    # the fp16 square transpose form agrees with the batched one
    src = rng.integers(0, 256, 9 * 9 * 2, dtype=np.uint8)
    assert np.array_equal(F.transpose(src, 9), F.transpose_batched(src, 1, 9, 9, 2))


def test_shard_pack_exchange_reassembles_the_transpose():
    """The pack of a row-sharded transpose, followed by the exchange (GPU j receives
    block j of every GPU's pack), leaves on each GPU its row block of the transposed
    matrix: simulated for a 48 x 48 matrix over 4 GPUs with the oracle's copy."""
    n, g = 48, 4
    rows = n // g
    m = np.random.default_rng(11).integers(0, 1 << 16, (n, n), dtype=np.uint16)
    w = W.shard_pack(rows, n, g)
    Ls, Ld = O.parse(w.src_layout), O.parse(w.dst_layout)
    packs = []
    for i in range(g):
        block = np.ascontiguousarray(m[i * rows:(i + 1) * rows]).reshape(-1).view(np.uint8)
        dst = np.full(block.size, 0xA5, np.uint8)
        packs.append(O.copy(block, Ls, dst, Ld, 2).view(np.uint16).reshape(g, rows * rows))
    for j in range(g):
        # GPU j's share of the transposed matrix: rows [j*rows, (j+1)*rows), the
        # columns coming from GPU i at [i*rows, (i+1)*rows)
        got = np.concatenate([packs[i][j].reshape(rows, rows) for i in range(g)], axis=1)
        assert np.array_equal(got, m.T[j * rows:(j + 1) * rows])


# ---------------------------------------------------------------------------
# Complement, logical divide and products
# ---------------------------------------------------------------------------
def test_blocked_product_golden_shape():
    kv = {}
    with open(os.path.join(GOLDEN, "blocked_product.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k] = v.strip()
    R = O.blocked_product(O.parse(kv["tile"]), O.parse(kv["grid"]))
    assert O.fmt(R).split(":")[0] == kv["shape"]
    # every block position holds one whole copy of the tile, tiles laid out compactly
    offs = sorted(O.eval_indices(R, np.arange(O.size(R))).tolist())
    assert offs == list(range(320))
    for i in range(4):
        for j in range(8):
            assert O.eval_coord(R, ((i, 0), (j, 0))) == O.eval_coord(O.parse(kv["tile"]), (i, j))


def _nested_layout(rng):
    """Random injective layout whose leaves, sorted by stride, are disjoint and nested."""
    n = rng.randint(1, 3)
    leaves, cur = [], 1
    for _ in range(n):
        gap = rng.choice([1, 1, 2, 3])
        d = cur * gap
        e = rng.randint(2, 4)
        leaves.append((e, d))
        cur = e * d
    rng.shuffle(leaves)
    return O.Layout(tuple(e for e, _ in leaves), tuple(d for _, d in leaves)) if n > 1 else O.Layout(*leaves[0])


def test_complement_fills_the_gaps():
    rng = random.Random(61)
    assert O.fmt(O.complement(O.parse("(4,8):(1,4)"), 64)) == "2:32"
    assert O.fmt(O.complement(O.parse("4:2"), 24)) == "(2,3):(1,8)"
    for _ in range(500):
        A = _nested_layout(rng)
        M = O.cosize(A) * rng.randint(1, 3) + rng.randint(0, 5)
        C = O.complement(A, M)
        cat = O.Layout((A.shape, C.shape), (A.stride, C.stride))
        offs = sorted(O.eval_indices(cat, np.arange(O.size(cat))).tolist())
        assert offs == list(range(len(offs))), (A, M)  # a bijection onto a prefix
        assert len(offs) >= M
    with pytest.raises(OL.NotRepresentable):
        O.complement(O.parse("(2,2):(1,3)"), 12)  # 3 is not a multiple of 2*1


def test_logical_divide_rearranges():
    rng = random.Random(62)
    assert O.fmt(O.logical_divide(O.parse("24:1"), O.parse("4:2"))) == "(4,(2,3)):(2,(1,8))"
    hits = 0
    for _ in range(500):
        B = _nested_layout(rng)
        A = O.Layout(O.cosize(B) * rng.randint(1, 3), rng.choice([1, 2]))
        try:
            R = O.logical_divide(A, B)
        except OL.NotRepresentable:
            continue
        hits += 1
        if O.size(R) == O.size(A):  # the tiles and the rest cover A exactly once
            assert sorted(O.eval_indices(R, np.arange(O.size(R))).tolist()) == \
                sorted(O.eval_indices(A, np.arange(O.size(A))).tolist())
        tile = O.Layout(R.shape[0], R.stride[0])
        assert np.array_equal(O.eval_indices(tile, np.arange(O.size(B))), O.compose_table(A, B))
    assert hits > 300


def test_logical_product_repeats():
    rng = random.Random(63)
    hits = 0
    for _ in range(300):
        A, B = _nested_layout(rng), _nested_layout(rng)
        try:
            R = O.logical_product(A, B)
        except OL.NotRepresentable:
            continue
        hits += 1
        assert O.Layout(R.shape[0], R.stride[0]) == A
        assert O.is_injective_bruteforce(R)
        # repetition r of A sits at an offset that A itself never reaches
        k = np.arange(O.size(R))
        offs = O.eval_indices(R, k)
        first = offs[: O.size(A)]
        for r in range(1, O.size(B)):
            rep = offs[r * O.size(A):(r + 1) * O.size(A)]
            assert not set(rep.tolist()) & set(first.tolist())
        BP_ok = len(O.top_modes(A)) == len(O.top_modes(B))
        if BP_ok:
            P = O.blocked_product(A, B)
            assert sorted(O.eval_indices(P, k).tolist()) == sorted(offs.tolist())
    assert hits > 100


# ---------------------------------------------------------------------------
# Access-pattern checks (bank conflicts, cache lines)
# ---------------------------------------------------------------------------
def test_bank_conflicts_of_a_column_read():
    # [print_layout page, section 4.3]: 32 threads reading one column of 8-wide
    # row-major rows.  The page calls this 32-way; with 32 banks of 4 bytes the rows
    # are 32 bytes apart, so offsets 8t fall on banks 0, 8, 16, 24: 8-way.
    col = O.parse("32:8")                                  # thread t -> row t, column 0
    assert O.bank_ways(col, 4) == 8
    # [section 5.2]: padding the row to 9 elements spreads the column over all banks
    assert O.bank_ways(O.parse("32:9"), 4) == 1
    # [section 4.3]: the XOR swizzle row*8 + (col ^ row) on the same column access
    sw = O.parse("Sw<3,0,3> o (32,8):(8,1)")
    assert O.bank_ways(sw, 4) == 4
    # a row read is conflict-free; the same address is a broadcast, not a conflict
    assert O.bank_ways(O.parse("32:1"), 4) == 1
    assert O.bank_ways(O.parse("32:0"), 4) == 1


def test_lines_touched():
    # [print_layout page, section 5.1]: adjacent threads on adjacent addresses
    assert O.lines_touched(O.parse("64:1"), 4) == 2          # 256 contiguous bytes
    assert O.lines_touched(O.parse("64:32"), 4) == 64        # one line per thread
    assert O.lines_touched(O.parse("(8,8):(1,1024)"), 16) == 8  # 8 rows of 128 bytes
    # brute-force cross-check with a different counting
    rng = random.Random(81)
    for _ in range(200):
        L = _rand_layout(rng, max_stride=40, allow_zero=False)
        if O.size(L) < 8:
            continue
        eb = rng.choice([1, 2, 4, 16])
        n = min(O.size(L), 64)
        byts = {O.eval_index(L, t) * eb + i for t in range(n) for i in range(eb)}
        assert O.lines_touched(L, eb, lanes=n) == len({b // 128 for b in byts})


def test_lds_cycles_closed_form():
    # A phase of P consecutive lanes at word stride s > 0 visits banks s*t mod B, which
    # repeat every B/gcd(s,B) lanes on distinct words: ceil(P*gcd(s,B)/B) ways.
    for B in (32, 64):
        for P in (8, 16, 32, 64):
            for s in range(1, 70):
                ways = -(-P * math.gcd(s, B) // B)
                cyc, ph, worst, hist = O.lds_cycles(O.Layout((64,), (s,)), 4, 64, B, P)
                assert (ph, worst, cyc) == (64 // P, ways, ways * (64 // P)), (B, P, s)
                assert sum(hist) == P and max(hist) == worst
    # all lanes on one word: a broadcast
    assert O.lds_cycles(O.parse("64:0"), 4, 64, 32, 32)[:3] == (2, 2, 1)


def test_lds_cycles_pins_and_invariants():
    # the page's column read: one phase of 32 lanes on 32 banks
    assert O.lds_cycles(O.parse("32:8"), 4, 32, 32, 32)[:3] == (8, 1, 8)
    assert O.lds_cycles(O.parse("32:9"), 4, 32, 32, 32)[:3] == (1, 1, 1)
    # wide elements: a 16-byte element covers 4 consecutive banks
    assert O.lds_cycles(O.parse("16:1"), 16, 16, 64, 16)[:3] == (1, 1, 1)
    assert O.lds_cycles(O.parse("16:4"), 16, 16, 64, 16)[:3] == (4, 1, 4)
    rng = random.Random(82)
    for _ in range(300):
        L = _rand_layout(rng, max_stride=70, allow_zero=True)
        n = O.size(L)
        if n < 4:
            continue
        eb = rng.choice([1, 2, 4, 8, 16])
        lanes = min(n, 64)
        B = rng.choice([32, 64])
        P = rng.choice([4, 8, 16, 32, 64])
        cyc, ph, worst, hist = O.lds_cycles(L, eb, lanes, B, P)
        assert ph == -(-lanes // P)
        assert ph <= cyc <= ph * P * max(1, -(-eb // 4) + 1)
        # one phase covering every lane is the plain bank_ways count
        assert O.lds_cycles(L, eb, lanes, B, lanes)[2] == O.bank_ways(L, eb, lanes, B)
        # permuting lanes inside each phase leaves the count unchanged
        offs = [O.eval_index(L, t) for t in range(lanes)]
        perm = []
        for p in range(0, lanes, P):
            grp = list(range(p, min(lanes, p + P)))
            rng.shuffle(grp)
            perm += grp
        # a table layout is not a layout: recount directly from the permuted offsets
        tot = 0
        for p in range(0, lanes, P):
            per = {}
            for t in perm[p:p + P]:
                a = offs[t] * eb
                for w in range(a // 4, (a + eb - 1) // 4 + 1):
                    per.setdefault(w % B, set()).add(w)
            tot += max(len(v) for v in per.values())
        assert tot == cyc


def test_access_report_adjacency_and_lines():
    r = O.access_report(O.parse("64:1"), 4, 64, 32, 32)
    assert r["adjacent"] and r["first_gap"] == -1 and r["lines"] == r["min_lines"] == 2
    assert r["conflict_cycles"] == 0
    # the strip-mined thread map (Pitch 8, Strips 4, kRow 16): runs of 8 lanes
    r = O.access_report(O.stripmined_layout(8, 4, 16, 64), 2, 64, 32, 32)
    assert not r["adjacent"] and r["first_gap"] == 7
    # 2-byte elements: runs of 16 bytes every 32 bytes, then the next group 1 KiB on
    assert r["lines"] == 2 and r["min_lines"] == 1
    # 16-byte elements: each run of 8 lanes fills one 128-byte line exactly
    r = O.access_report(O.stripmined_layout(8, 4, 16, 64), 16, 64, 64, 16)
    assert r["lines"] == r["min_lines"] == 8
    # a broadcast: every lane on one element
    r = O.access_report(O.parse("64:0"), 8, 64, 64, 32)
    assert r["lines"] == r["min_lines"] == 1 and r["first_gap"] == 0


@pytest.mark.parametrize("name", ["threadmap_p8_s4_k16.txt", "threadmap_p8_s2_k16.txt"])
def test_thread_offset_table_matches_golden(name):
    h, rows = _golden(name)
    kv = dict(x.split("=") for x in h["map"].split()[1:])
    p, s, k, t = (int(kv[x]) for x in ("pitch", "strips", "krow", "threads"))
    table = O.thread_offset_table(O.stripmined_layout(p, s, k, t), t).split("\n")
    assert len(table) == t
    got = {}
    for line in table:
        m = re.fullmatch(r"thread +(\d+) -> offset +(\d+)", line)
        got[int(m.group(1))] = int(m.group(2))
    assert len({len(x) for x in table}) == 1          # fixed-width columns
    for r in rows:
        t0, t1, o0 = (int(x) for x in r.split())
        for tid in range(t0, t1 + 1):
            assert got[tid] == o0 + tid - t0
