"""Host side of the C ABI (no GPU): the library loads and exports what the header
declares, and its layout algebra and copy planner agree with the CPU oracle."""

import math
import os
import random
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O
from oracle import layout as OL
import workloads as W

lr = pytest.importorskip("layout_remapping_copy_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(lr.LIB_PATH):
        pytest.skip("library not built")


def _same(Lc, Lo):
    """C descriptor equals oracle layout: same leaves, same swizzle."""
    return Lc.leaves == O.flatten(Lo) and Lc.swizzle == Lo.swz


def _rand_layout(rng, max_leaves=4, max_ext=4, max_stride=16, swz_p=0.0, allow_zero=True):
    nl = rng.randint(1, max_leaves)
    ext = [rng.randint(1, max_ext) for _ in range(nl)]
    st = [rng.randint(0 if allow_zero else 1, max_stride) for _ in range(nl)]
    modes, i = [], 0
    while i < nl:
        j = rng.randint(i + 1, nl)
        modes.append((ext[i:j], st[i:j]))
        i = j

    def t(xs):
        return str(xs[0]) if len(xs) == 1 else "(" + ",".join(map(str, xs)) + ")"

    if len(modes) == 1 and len(modes[0][0]) == 1:
        text = f"{ext[0]}:{st[0]}"
    else:
        text = "(" + ",".join(t(m[0]) for m in modes) + "):(" + ",".join(t(m[1]) for m in modes) + ")"
    if rng.random() < swz_p:
        b = rng.randint(1, 2)
        text = f"Sw<{b},{rng.randint(0, 2)},{rng.randint(b, 3)}> o " + text
    return text


def test_exports_every_header_symbol():
    names = lr.header_symbols()
    assert len(names) >= 19
    h = lr.lib()
    for n in names:
        assert hasattr(h, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lr.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines() if " T " in line)
    assert exported == names


def test_binding_has_every_entry_point():
    """Each lr_X of the header has a Python function X in the binding."""
    from layout_remapping_copy_amd import binding as B
    for name in lr.header_symbols():
        assert callable(getattr(B, name[3:], None)), name
    assert lr.layout_format(lr.layout_parse("(4,2):(_2,_1)")) == "(4,2):(2,1)"
    assert (lr.size("(4,2):(2,1)"), lr.cosize("(4,2):(2,1)")) == (8, 8)
    lr.layout_validate("Sw<3,3,3> o (64,64):(64,1)")
    assert lr.version() and lr.last_hip_error() == ""
    big = "(" + ",".join(["3"] * 16) + "):(" + ",".join([str(10 ** 18 + i) for i in range(16)]) + ")"
    with pytest.raises(lr.LayoutRemapError):
        lr.layout_validate(big)   # the largest offset overflows int64


def test_parse_format_pins():
    for t in ["(4,2):(2,1)", "((4,2),(2,4)):((2,16),(1,8))", "Sw<3,3,3> o ((128,32),(64,64)):((64,524288),(1,8192))",
              "8:1", "(4,2,2):(8,2,1)", "((4,8),2):((16,1),8)"]:
        assert str(lr.parse(t)) == t
    assert str(lr.parse("(4,2,2):(_8,_2,_1)")) == "(4,2,2):(8,2,1)"
    assert str(lr.parse("Sw<3,0,3> ∘ (8,8):(8,1)")) == "Sw<3,0,3> o (8,8):(8,1)"
    L = lr.parse("(((2,2),3),5):(((1,2),4),12)")
    assert L.leaves == [(2, 1), (2, 2), (3, 4), (5, 12)] and L.mode_end == [3, 4]
    for bad, code in [("(4,2):(1)", lr.binding.ERR_INVALID), ("(4,2):(1,-1)", lr.binding.ERR_INVALID),
                      ("(0,2):(1,1)", lr.binding.ERR_INVALID), ("Sw<3,0,2> o 8:1", lr.binding.ERR_SWIZZLE),
                      ("8:1 junk", lr.binding.ERR_INVALID), ("(1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17):"
                                                              "(1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17)",
                                                              lr.binding.ERR_INVALID)]:
        with pytest.raises(lr.LayoutRemapError) as e:
            lr.parse(bad)
        assert e.value.code == code, bad
    with pytest.raises(lr.LayoutRemapError) as e:
        lr.parse("(4294967296,4294967296,4294967296):(1,1,1)")
    assert e.value.code == lr.binding.ERR_OVERFLOW


def test_parse_matches_oracle_random():
    rng = random.Random(17)
    for _ in range(2000):
        t = _rand_layout(rng, max_leaves=6, swz_p=0.3)
        Lc, Lo = lr.parse(t), O.parse(t)
        assert _same(Lc, Lo), t
        assert Lc.size == O.size(Lo)
        if Lo.swz is None:
            assert Lc.cosize == O.cosize(Lo)
        else:
            assert Lc.cosize >= O.cosize(Lo)
        assert str(lr.parse(str(Lc))) == str(Lc)


def test_coalesce_matches_oracle():
    rng = random.Random(18)
    assert str(lr.coalesce("(8,8):(1,8)")) == "64:1"
    for _ in range(2000):
        t = _rand_layout(rng, max_leaves=6, swz_p=0.3)
        assert _same(lr.coalesce(t), O.coalesce(O.parse(t))), t


def test_composition_matches_oracle():
    assert str(lr.composition("(8,8):(1,9)", "((4,8),2):((16,1),8)")) == "((4,8),2):((18,1),9)"
    assert str(lr.composition("(8,8):(1,8)", "((4,8),2):((16,1),8)")) == "((4,8),2):((16,1),8)"
    rng = random.Random(19)
    agree = 0
    for _ in range(4000):
        ta = _rand_layout(rng, swz_p=0.2)
        tb = _rand_layout(rng, max_stride=6, swz_p=0.05)
        try:
            want = O.compose(O.parse(ta), O.parse(tb))
        except OL.NotRepresentable:
            want = None
        try:
            got = lr.composition(ta, tb)
        except lr.LayoutRemapError as e:
            assert e.code == lr.binding.ERR_NOT_REPRESENTABLE
            got = None
        assert (got is None) == (want is None), (ta, tb)
        if got is not None:
            agree += 1
            assert _same(got, want), (ta, tb, str(got), O.fmt(want))
    assert agree > 1000


def test_right_inverse_matches_oracle():
    assert str(lr.right_inverse("((4,8),2):((16,1),8)")) == "(8,2,4):(4,32,1)"
    rng = random.Random(20)
    for _ in range(2000):
        t = _rand_layout(rng)
        assert _same(lr.right_inverse(t), O.right_inverse(O.parse(t))), t
    with pytest.raises(lr.LayoutRemapError):
        lr.right_inverse("Sw<1,0,1> o 4:1")


def test_zipped_divide_matches_oracle():
    Z = lr.zipped_divide("(128,128):(1,128)", (4, 8))
    assert str(Z) == "((4,8),(32,16)):((1,128),(4,1024))"
    rng = random.Random(21)
    for _ in range(500):
        r, c = rng.choice([2, 4, 6, 8, 12]), rng.choice([2, 3, 4, 8])
        t = f"({r},{c}):({rng.randint(0, 5)},{rng.randint(1, 20)})"
        tr = rng.choice([x for x in (1, 2, 3, 4) if r % x == 0])
        tc = rng.choice([x for x in (1, 2, 4) if c % x == 0])
        got = lr.zipped_divide(t, (tr, tc))
        want = O.zipped_divide(O.parse(t), (tr, tc))
        assert got.leaves == O.flatten(want)
    with pytest.raises(lr.LayoutRemapError):
        lr.zipped_divide("(6,4):(1,6)", (4,))


def _mode_ends(Lo):
    ends, n = [], 0
    for m in O.top_modes(Lo):
        n += len(O.flatten(m))
        ends.append(n)
    return ends


def test_slice_matches_oracle():
    # [CuTe algebra page, section 3.2]: tile (3,5) of the zipped_divide
    Z = lr.zipped_divide("(128,128):(1,128)", (4, 8))
    T, off = lr.slice(Z, (-1, 3 + 32 * 5))
    assert (str(T), off) == ("(4,8):(1,128)", 5132)
    T2, off2 = lr.slice(Z, (-1, -1, 3, 5))  # one entry per leaf
    assert (str(T2), off2) == ("(4,8):(1,128)", 5132)
    rng = random.Random(33)
    runs = 0
    for _ in range(1500):
        t = _rand_layout(rng, max_leaves=5, swz_p=0.2)
        Lo, Lc = O.parse(t), lr.parse(t)
        top = O.top_modes(Lo)
        per_mode = rng.random() < 0.5
        if per_mode:
            coord = [None if rng.random() < 0.5 else rng.randrange(O.size(m)) for m in top]
            oc = tuple(coord) if not isinstance(Lo.shape, int) else coord[0]
        else:
            # one entry per leaf; the oracle gets the same coordinate, nested like the shape
            coord = [None if rng.random() < 0.5 else rng.randrange(n) for n, _ in O.flatten(Lo)]
            it = iter(coord)

            def nest(shape):
                return next(it) if isinstance(shape, int) else tuple(nest(x) for x in shape)

            oc = nest(Lo.shape)
            if isinstance(Lo.shape, int):
                oc = (oc,)
        try:
            want = O.slice_layout(Lo, oc)
        except OL.NotRepresentable:
            want = None
        try:
            got = lr.slice(Lc, coord)
        except lr.LayoutRemapError as e:
            assert e.code == lr.binding.ERR_NOT_REPRESENTABLE, (t, coord)
            got = None
        assert (got is None) == (want is None), (t, coord)
        if got is None:
            continue
        (Sc, oc_), (So, oo) = got, want
        assert oc_ == oo and _same(Sc, So), (t, coord, str(Sc), O.fmt(So))
        # the same top-level modes
        assert Sc.mode_end == _mode_ends(So), (t, coord, str(Sc), O.fmt(So))
        runs += 1
    assert runs > 1200
    E = lr.binding
    for bad in ((-1,), (0, 0, 0, 0, 0), (-1, 512)):
        with pytest.raises(lr.LayoutRemapError) as e:
            lr.slice(Z, bad)
        assert e.value.code == E.ERR_INVALID, bad
    with pytest.raises(lr.LayoutRemapError) as e:
        lr.slice("Sw<3,3,3> o (64,64):(64,1)", (1, -1))
    assert e.value.code == E.ERR_NOT_REPRESENTABLE


def _nested_text(rng):
    n = rng.randint(1, 3)
    leaves, cur = [], 1
    for _ in range(n):
        d = cur * rng.choice([1, 1, 2, 3])
        e = rng.randint(2, 4)
        leaves.append((e, d))
        cur = e * d
    rng.shuffle(leaves)
    if n == 1:
        return f"{leaves[0][0]}:{leaves[0][1]}"
    return "(" + ",".join(str(e) for e, _ in leaves) + "):(" + ",".join(str(d) for _, d in leaves) + ")"


def test_complement_divide_products_match_oracle():
    assert str(lr.complement("(4,8):(1,4)", 64)) == "2:32"
    assert str(lr.logical_divide("24:1", "4:2")) == "(4,(2,3)):(2,(1,8))"
    assert str(lr.blocked_product("(4,8):(1,4)", "(2,5):(1,2)")) == "((4,2),(8,5)):((1,32),(4,64))"
    rng = random.Random(71)
    counts = [0, 0, 0, 0]
    for _ in range(1500):
        ta, tb = _nested_text(rng), _nested_text(rng)
        A, B = O.parse(ta), O.parse(tb)
        M = O.cosize(A) * rng.randint(1, 3) + rng.randint(0, 4)
        for i, (fo, fc) in enumerate([(lambda: O.complement(A, M), lambda: lr.complement(ta, M)),
                                      (lambda: O.logical_divide(O.Layout(O.cosize(B) * 2, 1), B),
                                       lambda: lr.logical_divide(f"{O.cosize(B) * 2}:1", tb)),
                                      (lambda: O.logical_product(A, B), lambda: lr.logical_product(ta, tb)),
                                      (lambda: O.blocked_product(A, B), lambda: lr.blocked_product(ta, tb))]):
            try:
                want = fo()
            except (OL.NotRepresentable, ValueError):
                want = None
            try:
                got = fc()
            except lr.LayoutRemapError as e:
                assert e.code in (lr.binding.ERR_NOT_REPRESENTABLE, lr.binding.ERR_INVALID)
                got = None
            assert (got is None) == (want is None), (i, ta, tb)
            if got is not None:
                counts[i] += 1
                assert got.leaves == O.flatten(want), (i, ta, tb, str(got), O.fmt(want))
    assert min(counts) > 100, counts


def test_is_injective_matches_oracle():
    assert not lr.is_injective("((4,2),(2,4)):((2,16),(1,8))")
    assert lr.is_injective("(4,2,2):(8,2,1)")
    assert lr.is_injective("(3,2):(2,3)")  # small: exact
    rng = random.Random(22)
    for _ in range(3000):
        t = _rand_layout(rng, max_leaves=5, swz_p=0.3)
        assert lr.is_injective(t) == O.is_injective(O.parse(t)), t
    for name in W.FULL:
        w = W.full(name)
        assert lr.is_injective(w.dst_layout) == O.is_injective(O.parse(w.dst_layout))
    # above 2^20 elements: separated leaves and an exact prefix, as the oracle
    M = (1 << 22) + 3
    for t, want in ((f"(3,2,{M}):(2,3,8)", True), (f"(3,2,{M}):(2,2,8)", False), (f"(2,{M}):(0,1)", False),
                    (f"Sw<2,1,3> o ({M},3,2):(8,2,3)", True), (f"({1 << 21},2):(1,{(1 << 21) - 1})", False),
                    (f"({1 << 21},2):(1,{1 << 21})", True), (f"({1 << 13},{1 << 12}):(1,{(1 << 13) - 1})", False),
                    ("(1024,3):(1048576,1048577)", True), ("(1024,3):(1048576,1048576)", False),
                    (f"(1024,3,{M}):(1048576,1048577,{1 << 31})", True)):
        assert lr.is_injective(t) == want == O.is_injective(O.parse(t)), t
    rng = random.Random(23)
    for _ in range(200):  # a small random head times a large separated tail
        head = _rand_layout(rng, max_leaves=3, max_ext=5, max_stride=9)
        Lh = O.parse(head)
        span = O.cosize(Lh)
        big = f"{(1 << 20) // O.size(Lh) + 7}:{span}"
        t = f"({head.split(':')[0]},{big.split(':')[0]}):({head.split(':')[1]},{big.split(':')[1]})"
        assert lr.is_injective(t) == O.is_injective(O.parse(t)) == O.is_injective_bruteforce(Lh), t


def test_thread_map_matches_oracle():
    for p, s, k, t in [(8, 4, 16, 64), (8, 2, 16, 32), (4, 3, 17, 100), (32, 1, 64, 256)]:
        L = lr.thread_map(p, s, k, t)
        assert L.leaves == O.flatten(O.stripmined_layout(p, s, k, t))
        B = lr.thread_map(p, 0, k, t)
        assert B.leaves == O.flatten(O.pitch_linear_layout(p, k, t))


def _rank2_text(rng, swz_p=0.3):
    def mode():
        k = rng.randint(1, 2)
        e = [rng.randint(1, 5) for _ in range(k)]
        d = [rng.randint(0, 40) for _ in range(k)]
        if k == 1:
            return str(e[0]), str(d[0])
        return "(" + ",".join(map(str, e)) + ")", "(" + ",".join(map(str, d)) + ")"
    (e0, d0), (e1, d1) = mode(), mode()
    text = f"({e0},{e1}):({d0},{d1})"
    if rng.random() < swz_p:
        b = rng.randint(1, 3)
        text = f"Sw<{b},{rng.randint(0, 2)},{rng.randint(b, 4)}> o " + text
    return text


def test_print_layout_and_table_match_oracle():
    # [print_layout page, section 3.1]: the 4x2 row-major example
    assert lr.layout_print("(4,2):(2,1)") == "(4,2):(2,1)\n0 1\n2 3\n4 5\n6 7\n"
    rng = random.Random(91)
    for _ in range(300):
        t = _rank2_text(rng)
        assert lr.layout_print(t) == O.print_layout(O.parse(t)) + "\n", t
        n = rng.randint(1, O.size(O.parse(t)))
        assert lr.layout_print_table(t, n) == O.thread_offset_table(O.parse(t), n) + "\n", t
    # the ThreadMap page's strip-mined map, 64 threads
    L = lr.thread_map(8, 4, 16, 64)
    assert lr.layout_print_table(L, 64) == O.thread_offset_table(O.stripmined_layout(8, 4, 16, 64), 64) + "\n"
    for bad in ("8:1", "(2,2,2):(1,2,4)"):
        with pytest.raises(lr.LayoutRemapError):
            lr.layout_print(bad)
    with pytest.raises(lr.LayoutRemapError):
        lr.layout_print_table("8:1", 9)
    with pytest.raises(lr.LayoutRemapError):
        lr.layout_print("(1024,1025):(1,1024)")   # more than 2^20 cells
    # capacity protocol: too small a buffer reports the size and writes nothing
    import ctypes
    need = ctypes.c_size_t()
    buf = ctypes.create_string_buffer(b"x" * 8)
    rc = lr.lib().lr_layout_print(ctypes.byref(lr.parse("(4,2):(2,1)").c), buf, 8, ctypes.byref(need))
    assert rc == lr.binding.ERR_CAPACITY and need.value == len("(4,2):(2,1)\n0 1\n2 3\n4 5\n6 7\n") + 1
    assert buf.raw[:8] == b"x" * 8


def test_access_check_matches_oracle():
    rng = random.Random(92)
    for _ in range(600):
        t = _rand_layout(rng, max_leaves=4, max_ext=6, max_stride=70, swz_p=0.3)
        Lo = O.parse(t)
        n = O.size(Lo)
        lanes = rng.randint(1, min(64, n))
        eb = rng.choice([1, 2, 4, 8, 16])
        op = rng.choice(["read", "write", "custom", "custom"])
        if op != "custom":
            banks = lpp = 0
        else:
            banks, lpp = rng.choice([32, 64, 17]), rng.choice([1, 8, 16, 32, 64])
        line = rng.choice([0, 64, 128, 256])
        r = lr.access_check(t, eb, lanes, op, banks, lpp, line)
        if op == "read":
            banks, lpp = {1: (32, 32), 2: (32, 32), 4: (32, 32), 8: (64, 32), 16: (64, 16)}[eb]
        elif op == "write":
            banks, lpp = {1: (32, 32), 2: (32, 32), 4: (32, 32), 8: (32, 16), 16: (32, 8)}[eb]
        want = O.access_report(Lo, eb, lanes, banks, lpp, line or 128)
        assert (r["banks"], r["lanes_per_phase"], r["line_bytes"]) == (banks, lpp, line or 128)
        for k in ("offsets", "cycles", "phases", "ways_max", "conflict_cycles", "bank_words", "lines",
                  "min_lines", "adjacent", "first_gap"):
            assert r[k] == want[k], (t, eb, lanes, banks, lpp, k, r[k], want[k])
    # the print_layout page's column read under its own warp model, and padded
    assert lr.access_check("32:8", 4, 32, "custom", 32, 32)["ways_max"] == 8
    assert lr.access_check("32:9", 4, 32, "custom", 32, 32)["conflict_cycles"] == 0
    for args in [("8:1", 4, 9), ("64:1", 4, 65), ("64:1", 3, 64), ("64:1", 4, 64, "custom", 32, 0),
                 ("64:1", 4, 64, "custom", 65, 8), ("64:1", 4, 64, "read", 32, 32), ("64:1", 4, 64, "read", 0, 0, -1),
                 ("2:4611686018427387903", 16, 2)]:
        with pytest.raises(lr.LayoutRemapError):
            lr.access_check(*args)
    import ctypes
    r = lr.binding.lr_access_report()
    assert lr.lib().lr_access_check(ctypes.byref(lr.parse("64:1").c), 4, 64, 3, 0, 0, 0, ctypes.byref(r)) == \
        lr.binding.ERR_INVALID


TILE_SHAPES = [(16, 16), (32, 16), (16, 32), (32, 32), (32, 8), (64, 8), (64, 16)]


@pytest.mark.parametrize("ta,tb", TILE_SHAPES)
def test_transpose_lds_tile_accesses_conflict_free(ta, tb):
    """The transpose kernel's LDS tile is C tile[TA*V][TB] with C = V elements of EB
    bytes; thread tid = alpha + TA*beta stores its i-th transposed row at
    tile[V*alpha + i][beta ^ (alpha % TB)], and after the barrier thread tid loads
    tile[row][c ^ ((row / V) % TB)] with c = tid % TB, row = tid / TB (+ a multiple of
    NT/TB).  For wave 0 and i = 0 the store is the layout
    Sw<log2 TB, 0, log2(V*TB)> o (min(TA,64), 64/TA):(V*TB, 1) over the lane, the load
    Sw<log2 TB, 0, log2(TB*V)> o 64:1 (other waves and i only XOR or shift the
    offsets by constants that keep the bank pattern).  With 16-byte chunks both are conflict-free under the gfx950
    model; the hardware counter shows 0 conflict cycles for these kernels."""
    for V in (1, 4, 8, 16):
        la = min(ta, 64)
        lb = 64 // la
        B, S = tb.bit_length() - 1, (V * tb).bit_length() - 1
        text = f"Sw<{B},0,{S}> o ({la},{lb}):({V * tb},1)" if lb > 1 else f"Sw<{B},0,{S}> o {la}:{V * tb}"
        rep = lr.access_check(text, 16, 64, "write")
        want = [(V * (t % ta)) * tb + ((t // ta) ^ ((t % ta) % tb)) for t in range(64)]
        assert rep["offsets"] == want, text
        assert rep["conflict_cycles"] == 0, (text, rep["conflict_cycles"])
        # the load: row = t / TB, so the XOR term takes the bits of t above TB*V
        load = [(t // tb) * tb + ((t % tb) ^ ((t // tb // V) % tb)) for t in range(64)]
        rep = lr.access_check(f"Sw<{B},0,{(tb * V).bit_length() - 1}> o 64:1", 16, 64, "read")
        assert rep["offsets"] == load
        assert rep["conflict_cycles"] == 0


@pytest.mark.parametrize("ta,tb", [(16, 16), (32, 16), (16, 32), (32, 32)])
def test_direct_load_transpose_lds_reads_conflict_free(ta, tb):
    """The direct-load transpose keeps source chunk (row r, column c) at LDS slot
    r*TA + (c ^ ((r/V) % 16)); lane tid = beta + TB*alpha reads rows V*beta + j of
    column alpha.  For wave 0 and j = 0 that is Sw<4,0,log2(V*TA)> o
    (TB,64/TB):(V*TA,1) over the lane (other waves and j XOR or shift by
    constants), conflict-free for 16-byte reads; the loads write 64 consecutive
    slots per wave."""
    for V in (1, 2, 4, 8, 16):
        if ta * tb * V * 16 > 160 * 1024:
            continue
        S = (V * ta).bit_length() - 1
        text = f"Sw<4,0,{S}> o ({tb},{64 // tb}):({V * ta},1)" if tb < 64 else f"Sw<4,0,{S}> o 64:{V * ta}"
        rep = lr.access_check(text, 16, 64, "read")
        want = [(V * (t % tb)) * ta + ((t // tb) ^ ((t % tb) % 16)) for t in range(64)]
        assert rep["offsets"] == want, text
        assert rep["conflict_cycles"] == 0, (text, rep["conflict_cycles"])
        assert lr.access_check("64:1", 16, 64, "write")["conflict_cycles"] == 0
        # every slot of the tile is written once: slot -> (row, column) is a bijection
        slots = set()
        for s_ in range(tb * V * ta):
            r, cs = divmod(s_, ta)
            c = cs ^ ((r // V) % 16)
            assert 0 <= c < ta
            slots.add((r, c))
        assert len(slots) == tb * V * ta


def test_channel_shuffle_lds_reads():
    """The de-interleave's lanes read LDS chunks l*C + j (16 bytes each): with C odd
    the plain slots are conflict-free under the gfx950 model, with C = 2, 4, 8 the
    kernel's Sw<4,0,4> on chunk slots makes them so, and its consecutive-chunk
    writes stay conflict-free.  C = 6 keeps a two-way conflict."""
    for c in (3, 5, 7):
        assert lr.access_check(f"64:{c}", 16, 64, "read")["conflict_cycles"] == 0, c
    for c in (2, 4, 8):
        assert lr.access_check(f"64:{c}", 16, 64, "read")["conflict_cycles"] > 0, c
        assert lr.access_check(f"Sw<4,0,4> o 64:{c}", 16, 64, "read")["conflict_cycles"] == 0, c
    assert lr.access_check("Sw<4,0,4> o 64:1", 16, 64, "write")["conflict_cycles"] == 0
    assert lr.access_check("64:6", 16, 64, "read")["conflict_cycles"] == 4


def test_fast_paths_touch_the_fewest_lines():
    """Per wave instruction, in 16-byte chunks (print_layout page, section 6.4: adjacent
    lanes on adjacent addresses).  Transpose (fp16 8192^2, 32 x 32 chunks, V = 8):
    a load instruction has lane (alpha, beta) = (l % 32, l / 32) read source row
    b0 + 8*beta + j at chunk alpha, i.e. (32,2):(1,8*1024) chunks with a 1024-chunk
    pitch; a store instruction has lane l write chunk l % 32 of destination row
    a0 + l / 32 + 32*k, i.e. (32,2):(1,1024).  Vector path: 64 consecutive units.
    Staged path (padded tiles): lane l stores chunk 16*tile + c = l of the compact
    tiles, again 64:1.
    Each touches exactly as many 128-byte lines as its bytes need."""
    for text in ("(32,2):(1,8192)", "(32,2):(1,1024)", "64:1"):
        r = lr.access_check(text, 16, 64, "read")
        assert r["lines"] == r["min_lines"] == 8, text
    # a 16-chunk-wide tile (the column-major interleave's 16 x 32): rows of 256 B
    r = lr.access_check("(16,4):(1,2048)", 16, 64, "read")
    assert r["lines"] == r["min_lines"] == 8
    # a strided pattern the planner avoids: one chunk per row
    r = lr.access_check("64:1024", 16, 64, "read")
    assert r["lines"] == 64 and r["min_lines"] == 8


@pytest.mark.parametrize("eb", [1, 2, 4, 8])
def test_element_transpose_lds_conflict_free(eb):
    """The element-granular transpose writes source rows into LDS rows of 256 bytes
    padded to PITCH (260 bytes, 264 for 8-byte elements) and reads one column per
    destination row: lane l reads row l, i.e. 64:(PITCH/EB) elements.  Both are
    conflict-free under the gfx950 model."""
    pitch = 256 + (8 if eb > 4 else 4)
    assert lr.access_check(f"64:{pitch // eb}", eb, 64, "read")["conflict_cycles"] == 0
    assert lr.access_check("64:1", eb, 64, "write")["conflict_cycles"] == 0
    # without the padding the column read would serialise
    assert lr.access_check(f"64:{256 // eb}", eb, 64, "read")["conflict_cycles"] > 0


def test_staged_gather_conflicts_match_the_counter():
    """The padded-tiles kernel gathers 4-byte words from LDS: lane l of a wave reads
    word 72*(l/16) + (c%8) + 9*(c/8) + 18x with c = l % 16 (16 lanes per tile, the
    tile's 72-word footprint with its pad word every 9th), i.e. the lane layout
    (8,2,4):(1,9,72) plus a constant.  The model gives 2 extra cycles per wave read;
    2^20 gather reads per launch then make 2,097,152 conflict cycles, the value
    SQ_LDS_BANK_CONFLICT shows for that kernel.  No per-tile stride removes them:
    each tile's 16 words leave a hole in its bank set, so two tiles in one phase
    always share a bank."""
    r = lr.access_check("(8,2,4):(1,9,72)", 4, 64, "read")
    assert (r["cycles"], r["phases"], r["conflict_cycles"]) == (4, 2, 2)
    assert (1 << 20) * r["conflict_cycles"] == 2097152
    for S in range(72, 72 + 64):
        assert lr.access_check(f"(8,2,4):(1,9,{S})", 4, 64, "read")["conflict_cycles"] == 2


def test_common_vector_sound_and_tight_on_workloads():
    rng = random.Random(23)
    for _ in range(1500):
        td = _rand_layout(rng, max_stride=12, swz_p=0.2, allow_zero=False)
        Ld = O.parse(td)
        ts = _rand_layout(rng, max_stride=12, allow_zero=False)
        if O.size(O.parse(ts)) != O.size(Ld):
            ts = f"{O.size(Ld)}:1"
        for eb in (1, 2, 4, 8):
            v = lr.max_common_vector(ts, td, eb)
            w = O.max_common_vector(O.parse(ts), Ld, eb)
            assert v <= w and w % v == 0, (ts, td, eb, v, w)
    for name, want in [("tile8x8", 1), ("transpose", 1), ("retile", 8), ("interleave", 1), ("interleave_cm", 1),
                       ("nhwc2nchw", 1), ("padtiles", 1), ("shard_pack", 1), ("rgb_nhwc2nchw", 1)]:
        w = W.small(name)
        v = lr.max_common_vector(w.src_layout, w.dst_layout, w.elem_bytes)
        assert v == want == O.max_common_vector(O.parse(w.src_layout), O.parse(w.dst_layout), w.elem_bytes)
    assert lr.max_common_vector("64:1", "64:1", 2) == 8
    assert lr.max_common_vector("(4,4):(1,5)", "(4,4):(1,4)", 4) == 1


EXPECTED_PATH = {"tile8x8": "alias", "transpose": "transpose", "retile": "vector", "interleave": "interleave",
                 "interleave_cm": "transpose", "nhwc2nchw": "transpose", "padtiles": "staged",
                 "shard_pack": "transpose", "rgb_nhwc2nchw": "deinterleave", "head_split": "vector"}


@pytest.mark.parametrize("name", list(W.FULL))
def test_plan_of_workloads(name):
    w = W.full(name)
    flags = lr.COPY_ORDERED_ALIAS if w.ordered_alias else 0
    p = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, w.elem_bytes, flags)
    assert p["path"] == EXPECTED_PATH[name]
    if name != "tile8x8":
        want = O.joint_flat(O.parse(w.src_layout), O.parse(w.dst_layout), sort_by_dst=True)
        # same modes; the vector path walks the modes after the first in source order
        assert p["joint"][0] == tuple(want[0]) and sorted(p["joint"]) == sorted(tuple(m) for m in want)
    if name in ("retile", "head_split"):  # tiles of 128- and 256-byte atoms
        assert p["vec_elems"] * w.elem_bytes == 16 and p["vector_order"] == 3


def test_plan_joint_matches_oracle_random():
    rng = random.Random(24)
    n = 0
    for _ in range(2000):
        ts = _rand_layout(rng, max_leaves=5, max_stride=40, allow_zero=False)
        Ls = O.parse(ts)
        exts = [e for e, _ in O.flatten(Ls)]
        rng.shuffle(exts)
        Ld = O.Layout(tuple(exts), tuple(rng.randint(1, 60) for _ in exts)) if len(exts) > 1 else O.Layout(exts[0], 1)
        if not O.is_injective(Ld):
            continue
        jm = O.joint_flat(Ls, Ld, sort_by_dst=True)
        if jm is None:  # no common refinement: generic cannot apply, dual does
            with pytest.raises(lr.LayoutRemapError):
                lr.copy_plan(ts, O.cosize(Ls), O.fmt(Ld), O.cosize(Ld), 4, lr.COPY_FORCE_PATH(lr.PATH_GENERIC))
            assert lr.copy_plan(ts, O.cosize(Ls), O.fmt(Ld), O.cosize(Ld), 4)["path"] == "dual"
            continue
        p = lr.copy_plan(ts, O.cosize(Ls), O.fmt(Ld), O.cosize(Ld), 4, lr.COPY_FORCE_PATH(lr.PATH_GENERIC))
        n += 1
        got = [m for m in p["joint"] if m[0] > 1]
        # the same modes, the first one first (the rest may be walked in source order)
        assert sorted(got) == sorted(tuple(m) for m in jm) and got[:1] == [tuple(m) for m in jm[:1]], (ts, O.fmt(Ld))
    assert n > 300


NT = {"load_policy": 2}     # streaming loads and stores (sc1 where the kernel has it)
PLAIN = {"load_policy": 0}  # ordinary loads and stores


def test_plan_streaming_default_and_tile_shapes():
    # non-temporal accesses from a 64 MiB footprint (source plus destination bytes)
    n = (32 << 20) // 4
    assert lr.copy_plan(f"{n}:1", n, f"{n}:1", n, 4)["streaming"]
    assert not lr.copy_plan(f"{n - 1}:1", n, f"{n - 1}:1", n, 4)["streaming"]
    assert not lr.copy_plan(f"{n}:1", n, f"{n}:1", n, 4, tuning=PLAIN)["streaming"]
    assert lr.copy_plan("64:1", 64, "64:1", 64, 4, tuning=NT)["streaming"]
    # the per-element and aliased fallbacks keep plain accesses, whatever is asked
    for t in (None, NT):
        p = lr.copy_plan("(6,4):(1,6)", 24, "(4,6):(1,4)", 24, 4, tuning=t)
        assert p["path"] == "dual" and not p["streaming"]
        p = lr.copy_plan("8:1", 8, "8:0", 1, 4, lr.COPY_ORDERED_ALIAS, tuning=t)
        assert p["path"] == "alias" and not p["streaming"]
    # transpose tiles: rows far apart -> 32 x 32 chunks (16 x 32 when 16 chunks
    # cover the contiguous extent), two register blocks a lane for 2-byte elements in
    # 32 x 32 chunks; a contiguous source block per tile -> 32 x 8
    want = {"transpose": (256, 256, 512), "interleave_cm": (128, 256, 512), "nhwc2nchw": (256, 64, 256)}
    for name, (ta, tb, block) in want.items():
        w = W.full(name)
        p = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, w.elem_bytes)
        assert p["path"] == "transpose" and p["streaming"]
        assert (p["tile_a"], p["tile_b"], p["block"]) == (ta, tb, block), name
    # fewer 32 x 32-chunk tiles than compute units: 32 x 8 chunks (the shard pack:
    # 128 -> 512 workgroups); 4096^2 fp16 fills the 256 units and keeps 32 x 32
    w = W.full("shard_pack")
    p = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, w.elem_bytes)
    assert (p["tile_a"], p["tile_b"], p["block"], p["grid"]) == (256, 64, 256, 512), p
    p = lr.copy_plan("(1024,8192):(8192,1)", 1 << 23, "(1024,8192):(1,1024)", 1 << 23, 2)
    assert (p["tile_a"], p["tile_b"], p["grid"]) == (256, 64, 512), p
    p = lr.copy_plan("(4096,4096):(4096,1)", 1 << 24, "(4096,4096):(1,4096)", 1 << 24, 2)
    assert (p["tile_a"], p["tile_b"], p["grid"]) == (256, 256, 256), p
    # 1-byte elements move in 8-byte chunks, 32 x 16 of them a tile (256 x 128 bytes)
    p = lr.copy_plan("(8192,8192):(8192,1)", 1 << 26, "(8192,8192):(1,8192)", 1 << 26, 1)
    assert (p["vec_elems"], p["tile_a"], p["tile_b"], p["block"]) == (8, 256, 128, 512), p
    # u8 4096^2 in 8-byte chunks: 32 x 16-chunk tiles of 256 x 128 bytes already make 512
    p = lr.copy_plan("(4096,4096):(4096,1)", 1 << 24, "(4096,4096):(1,4096)", 1 << 24, 1)
    assert (p["vec_elems"], p["tile_a"], p["tile_b"], p["grid"]) == (8, 256, 128, 512), p
    # 8-byte elements: 16 x 32 chunks; 16-byte elements: 64 x 16
    p = lr.copy_plan("(4096,8192):(8192,1)", 1 << 25, "(4096,8192):(1,4096)", 1 << 25, 8)
    assert (p["vec_elems"], p["tile_a"], p["tile_b"], p["block"]) == (2, 32, 64, 512), p
    p = lr.copy_plan("(4096,4096):(4096,1)", 1 << 24, "(4096,4096):(1,4096)", 1 << 24, 16)
    assert (p["vec_elems"], p["tile_a"], p["tile_b"], p["block"]) == (1, 64, 16, 1024), p
    # a whole destination-contiguous extent of 17-32 chunks whose rows are adjacent in the
    # destination (NCHW -> NHWC, 256 fp16 channels): 8 x 32 chunks, one contiguous
    # destination block per tile; 64 channels keep 32 x 8, and NHWC -> NCHW its 32 x 8
    p = lr.copy_plan("(128,3136,256):(802816,1,3136)", 128 * 3136 * 256, "(128,3136,256):(802816,256,1)",
                     128 * 3136 * 256, 2)
    assert (p["tile_a"], p["tile_b"], p["block"], p["grid"]) == (64, 256, 256, 128 * 49), p
    p = lr.copy_plan("(256,12544,64):(802816,1,12544)", 256 * 12544 * 64, "(256,12544,64):(802816,64,1)",
                     256 * 12544 * 64, 2)
    assert (p["tile_a"], p["tile_b"]) == (256, 64), p
    # whole matrices both ways (fp32 128 x 96, 4096 of them): the whole-block shape with more
    # lanes at work, 8 x 32 chunks (96 = 3 x 32 along a) over 32 x 8 (96 of 128 along a)
    p = lr.copy_plan("(128,96,4096):(96,1,12288)", 128 * 96 * 4096, "(128,96,4096):(1,128,12288)",
                     128 * 96 * 4096, 4)
    assert (p["path"], p["tile_a"], p["tile_b"]) == ("transpose", 32, 128), p
    w = W.full("nhwc2nchw")  # a whole 256-channel block each way only along a: 32 x 8
    p = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    assert (p["tile_a"], p["tile_b"]) == (256, 64), p


def test_plan_workgroup_order():
    """Transpose workgroup order: b-tiles fastest unless a pitch is power-of-two
    heavy (a multiple of 16 KiB, or a power of two from 4 KiB); then the diagonal
    with b fastest, or with a fastest for tiles with longer source rows and no more
    a-tiles than b-tiles.  A single a-tile keeps b fastest.  Chunk tiles within 64
    bytes of a multiple of 16 KiB count as power-of-two heavy, and take the diagonal
    with a fastest when every such pitch lies just past a multiple.  Element tiles (rows
    without aligned chunks) take the diagonal with b fastest up to 64 bytes past a
    multiple of 8 KiB, else a fastest with at least as many a-tiles as b-tiles."""

    def order(rows, cols, eb, tuning=None):
        p = lr.copy_plan(f"({cols},{rows}):(1,{cols})", rows * cols, f"({cols},{rows}):({rows},1)", rows * cols, eb,
                         tuning=tuning)
        assert p["path"] == "transpose"
        return p["order"]

    want = {(8192, 8192, 2): 4, (16384, 16384, 2): 4, (2048, 32768, 2): 4, (32768, 2048, 2): 4,
            (8192, 8256, 2): 4,  # destination pitch 16 KiB
            (11264, 11264, 2): 1, (12288, 12288, 2): 1, (8191, 8191, 2): 0, (6144, 6144, 4): 1,
            (16383, 4097, 2): 1, (4097, 16383, 2): 0,  # element tiles: 33 x 128 and 128 x 33 tiles
            (8184, 8184, 2): 4, (8256, 8256, 2): 1,  # near 16 KiB: just short of a multiple
            (8224, 8224, 2): 2, (4100, 4100, 4): 2, (16416, 16416, 2): 2,  # just past one: a fastest
            (16392, 8192, 2): 4,  # one pitch a multiple of 16 KiB, the other just past two
            (8193, 8193, 2): 4, (8196, 8196, 2): 4, (12289, 12289, 2): 4, (8188, 8188, 2): 0,  # past 8 KiB
            (8193, 4097, 4): 4, (4097, 2049, 2): 4,  # both pitches past 8 KiB, or one past and one small
            (6144, 6144, 1): 2, (11264, 11264, 1): 2, (8184, 8184, 1): 2,  # 1-byte, 8-byte chunks: order 2
            (8192, 8192, 1): 2,  # 256 x 128 tiles (8-byte chunks), 32 a-tiles <= 64 b-tiles
            (2048, 32768, 1): 4,  # 64 a-tiles > 8 b-tiles
            (8192, 4096, 8): 4,  # 8-byte elements: 32 x 64 tiles, not longer along a
            (4096, 4096, 16): 2,  # 16-byte elements: 64 x 16 tiles, 64 a-tiles <= 256 b-tiles
            (8192, 8192, 4): 4}
    for (rows, cols, eb), o in want.items():
        assert order(rows, cols, eb) == o, (rows, cols, eb)
    for name, o in (("transpose", 4), ("interleave_cm", 1), ("nhwc2nchw", 1)):
        w = W.full(name)
        assert lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, w.elem_bytes)["order"] == o, name
    assert lr.copy_plan("64:1", 64, "64:1", 64, 4)["order"] == -1
    assert order(8192, 8192, 2, {"tile_order": 3}) == 3
    assert order(8192, 8192, 2, {"tile_order": 0}) == 0


def test_plan_store_policy():
    """Streaming copies load and store non-temporally; the streaming stores of the
    LDS transpose, the vector path and the narrow interleave also carry the sc1 scope
    bit (buffer stores), only while a tile's (transpose) or the whole destination's
    span stays under 4 GiB (32-bit buffer offsets)."""
    def plan(name, tuning=None):
        w = W.full(name)
        flags = lr.COPY_ORDERED_ALIAS if w.ordered_alias else 0
        return lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, w.elem_bytes, flags, tuning=tuning)

    want = {"transpose": (2, 18), "interleave_cm": (2, 18), "nhwc2nchw": (2, 18), "interleave": (2, 18),
            "padtiles": (2, 2), "retile": (2, 18), "shard_pack": (0, 0), "tile8x8": (0, 0)}
    for name, pol in want.items():
        p = plan(name)
        assert (p["load_policy"], p["store_policy"]) == pol, (name, p["path"])
    assert plan("transpose", {"store_policy": 2})["store_policy"] == 2
    # the direct-load kernel keeps global stores
    assert plan("transpose", {"direct_loads": 1})["store_policy"] == 2
    # 16-byte elements, 16 x 16 tiles: the destination span of a tile is 15 rows of the
    # a-mode's destination stride
    for sd, pol in ((1 << 20, 18), ((1 << 32) // (15 * 16) - 16, 18), (1 << 25, 2)):
        p = lr.copy_plan("(16,64):(1,16)", 1024, f"(16,64):({sd},1)", 15 * sd + 64, 16, tuning=NT)
        assert p["path"] == "transpose" and p["tile_a"] == 16 and p["store_policy"] == pol, (sd, p)
    # element tiles (rows without aligned chunks) keep global stores
    p = lr.copy_plan("(301,517):(517,1)", 301 * 517, "(301,517):(1,301)", 301 * 517, 2, tuning=NT)
    assert p["store_policy"] == 2
    # the vector path and 16-byte generic units: stores from the destination base,
    # span under 4 GiB
    assert plan("retile", NT)["store_policy"] == 18
    for n, pol in (((1 << 28) - 1, 18), (1 << 28, 2)):
        p = lr.copy_plan(f"{n}:1", n, f"{n}:1", n, 16, tuning=NT)
        assert p["vec_elems"] * p["elem_bytes"] == 16 and p["store_policy"] == pol, (n, p)
    assert lr.copy_plan("4096:1", 4096, "4096:1", 4096, 4, lr.COPY_WIDE_INDEX, tuning=NT)["store_policy"] == 2
    assert plan("retile", {"store_policy": 2})["store_policy"] == 2
    # loads and stores apart: the vector path only
    p = plan("retile", {"load_policy": 2, "store_policy": 0})
    assert (p["load_policy"], p["store_policy"]) == (2, 0)
    with pytest.raises(lr.LayoutRemapError) as e:
        plan("transpose", {"load_policy": 2, "store_policy": 0})
    assert e.value.code == lr.binding.ERR_PATH


def test_transpose_blocks_plan():
    """transpose_blocks = 2 halves the lanes of the register-loaded LDS transpose for
    the same tile; direct loads, element tiles and odd b sides keep one block a lane.
    By default 1024-lane tiles of 2-byte elements take two blocks a lane, others one."""
    w = W.full("transpose")
    args = (w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    base = lr.copy_plan(*args, tuning={"transpose_blocks": 1})
    p = lr.copy_plan(*args, tuning={"transpose_blocks": 2})
    assert base["block"] == 1024 and p["block"] == 512 and lr.copy_plan(*args)["block"] == 512
    assert (p["tile_a"], p["tile_b"], p["grid"], p["order"]) == (base["tile_a"], base["tile_b"], base["grid"], base["order"])
    f32 = ("(8192,8192):(8192,1)", 1 << 26, "(8192,8192):(1,8192)", 1 << 26, 4)
    assert lr.copy_plan(*f32)["block"] == 1024 and lr.copy_plan(*f32, tuning={"transpose_blocks": 2})["block"] == 512
    cm = W.full("interleave_cm")  # 512-lane tiles keep one block a lane
    assert lr.copy_plan(cm.src_layout, cm.src_elems, cm.dst_layout, cm.dst_elems, 2)["block"] == 512
    assert lr.copy_plan(*args, tuning={"transpose_blocks": 2, "direct_loads": 1})["block"] == 1024
    for shape in range(9):
        p = lr.copy_plan(*args, tuning={"transpose_blocks": 2, "tile_shape": shape})
        blocks = p["tile_a"] * p["tile_b"] // p["vec_elems"] ** 2
        assert p["block"] == (blocks if shape == 7 else blocks // 2), shape  # 8 x 8 chunks: one wavefront
    odd = ("(8191,8191):(8191,1)", 8191 * 8191, "(8191,8191):(1,8191)", 8191 * 8191, 2)
    assert lr.copy_plan(*odd, tuning={"transpose_blocks": 2})["block"] == lr.copy_plan(*odd)["block"]


def test_tuning_overrides_are_checked():
    w = W.full("transpose")
    args = (w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    for bad in ({"load_policy": 1}, {"store_policy": 16}, {"tile_shape": 9}, {"tile_order": 10},
                {"units_per_lane": 2}, {"vector_order": 4}, {"gather_chunks": 3}, {"direct_loads": 2},
                {"pipeline_tiles": 1}, {"pipeline_tiles": 65}, {"pipeline_tiles": -2}, {"transpose_reads": 2},
                {"chunk_bytes": 4}, {"chunk_bytes": 0}, {"workgroup_lanes": 32}, {"workgroup_lanes": 512},
                {"batch_swizzle": 16}, {"batch_order": 2}, {"transpose_blocks": 0}, {"transpose_blocks": 3}):
        with pytest.raises(lr.LayoutRemapError) as e:
            lr.copy_plan(*args, tuning=bad)
        assert e.value.code == lr.binding.ERR_INVALID, bad
    with pytest.raises(KeyError):
        lr.copy_plan(*args, tuning={"no_such_knob": 1})
    # knobs of other paths are ignored; -1 everywhere is the planner's own plan
    assert lr.copy_plan(*args, tuning={"gather_chunks": 8, "vector_order": 0}) == lr.copy_plan(*args)
    assert lr.copy_plan(*args, tuning={k: -1 for k in lr.binding.TUNING_FIELDS}) == lr.copy_plan(*args)


def test_pipelined_transpose_plan():
    """pipeline_tiles: tile shapes whose two LDS tiles fit (16x16, 32x16, 16x32 chunks of
    16 bytes) take that many consecutive tiles per workgroup with direct loads; the
    grid is the tile count divided up; elsewhere the override is ignored."""
    w = W.full("transpose")
    args = (w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    for shape, tiles in ((0, 64 * 64), (1, 32 * 64), (2, 64 * 32)):
        base = lr.copy_plan(*args, tuning={"tile_shape": shape})
        assert base["grid"] == tiles and base["pipeline_tiles"] == 0
        for pipe in (2, 3, 7, 64):
            p = lr.copy_plan(*args, tuning={"tile_shape": shape, "pipeline_tiles": pipe})
            assert p["pipeline_tiles"] == pipe and p["direct"], (shape, pipe)
            assert p["grid"] == -(-tiles // pipe) and (p["tile_a"], p["tile_b"]) == (base["tile_a"], base["tile_b"])
    # 32x32 chunks: 128 KiB of LDS per tile, two do not fit
    assert lr.copy_plan(*args, tuning={"tile_shape": 3, "pipeline_tiles": 4})["pipeline_tiles"] == 0
    # not a transpose, or no full 16-byte chunks: ignored
    r = W.full("retile")
    ra = (r.src_layout, r.src_elems, r.dst_layout, r.dst_elems, 2)
    assert lr.copy_plan(*ra, tuning={"pipeline_tiles": 4}) == lr.copy_plan(*ra)
    odd = ("(520,263):(263,1)", 520 * 263, "(520,263):(1,520)", 520 * 263, 2)
    assert lr.copy_plan(*odd, tuning={"pipeline_tiles": 4})["pipeline_tiles"] == 0


def test_atom_tiles_plan():
    """Vector order 3 (tiles of atoms through LDS): the planner's choice when the common
    contiguous mode is an atom of 64-512 bytes continued by different modes in the
    source and the destination, each at least one tile (1 KiB runs, >= 4 atoms) long;
    the source order otherwise, also when order 3 is asked for."""
    w = W.full("retile")
    args = (w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    p = lr.copy_plan(*args)
    assert (p["path"], p["vector_order"], p["tile_a"], p["tile_b"]) == ("vector", 3, 8, 8)
    joint = p["joint"]
    assert joint[0] == (64, 1, 1)
    assert joint[p["a_mode"]][1] == 64 and joint[p["b_mode"]][2] == 64   # a continues the atom in src, b in dst
    assert p["grid"] == (64 // 8) * (128 // 8) * 32
    q = lr.copy_plan(*args, tuning={"vector_order": 1})
    assert q["vector_order"] == 1 and q["grid"] == 4096 * 4096 // 8 // 256
    # atom sizes: up to 64 bytes -> 16 atoms a side, up to 240 -> 8, from 256 -> 4; from
    # 256 bytes only atoms that are not whole 128-byte lines (order 1 otherwise); 32- and
    # 48-byte atoms reach the vector path as tiles of atoms only
    for eb, w_, T in ((2, 16, 16), (2, 24, 16), (1, 64, 16), (2, 40, 8), (2, 64, 8), (2, 112, 8), (8, 32, 4),
                      (2, 160, 4), (2, 192, 0), (16, 32, 0)):
        ts, td = f"({w_},40,50):(1,{w_},{40 * w_})", f"({w_},40,50):(1,{50 * w_},{w_})"
        r = lr.copy_plan(ts, 2000 * w_, td, 2000 * w_, eb)
        if T:
            assert r["path"] in ("vector", "generic") and r["vector_order"] == 3 and r["tile_a"] == T, (eb, w_, r)
        else:
            assert r["vector_order"] == 1, (eb, w_, r)
    # one side shorter than a tile, or a 16-byte atom: not tiles of atoms
    short = lr.copy_plan("(64,7,50):(1,64,448)", 64 * 350, "(64,7,50):(1,3200,64)", 64 * 350, 2,
                         tuning={"vector_order": 3})
    assert short["vector_order"] == 1
    small = lr.copy_plan("(8,40,50):(1,8,320)", 16000, "(8,40,50):(1,400,8)", 16000, 2)
    assert small["vector_order"] != 3


def test_transpose_reads_plan():
    """transpose_reads: the direct-load (or pipelined) LDS transpose of 2- or 1-byte
    elements in 16-byte chunks, tile shapes 0-3 (0-2 for 1-byte elements, whose 32 x 32
    chunk tile does not fit in LDS); ignored without direct loads or for other element
    sizes."""
    w = W.full("transpose")
    args = (w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    assert not lr.copy_plan(*args)["transpose_reads"]
    assert not lr.copy_plan(*args, tuning={"transpose_reads": 1})["transpose_reads"]  # no direct loads
    for shape in range(4):
        p = lr.copy_plan(*args, tuning={"transpose_reads": 1, "direct_loads": 1, "tile_shape": shape})
        assert p["transpose_reads"] and p["direct"] and p["tile_a"] == (16, 32, 16, 32)[shape] * 8, shape
    p = lr.copy_plan(*args, tuning={"transpose_reads": 1, "pipeline_tiles": 4, "tile_shape": 1})
    assert p["transpose_reads"] and p["pipeline_tiles"] == 4
    # 32 x 8 chunks (shape 4): the reads need 16 or 32 chunks on both sides
    assert not lr.copy_plan(*args, tuning={"transpose_reads": 1, "direct_loads": 1, "tile_shape": 4})["transpose_reads"]
    f32 = ("(4096,4096):(4096,1)", 4096 * 4096, "(4096,4096):(1,4096)", 4096 * 4096, 4)
    assert not lr.copy_plan(*f32, tuning={"transpose_reads": 1, "direct_loads": 1})["transpose_reads"]
    # 1-byte elements: 16-byte chunks (8-byte ones otherwise)
    u8 = ("(4096,4096):(4096,1)", 4096 * 4096, "(4096,4096):(1,4096)", 4096 * 4096, 1)
    assert lr.copy_plan(*u8)["vec_elems"] == 8 and not lr.copy_plan(*u8)["transpose_reads"]
    for shape, ta, tb in ((0, 16, 16), (1, 32, 16), (2, 16, 32), (3, 32, 16)):
        p = lr.copy_plan(*u8, tuning={"transpose_reads": 1, "direct_loads": 1, "tile_shape": shape})
        assert p["transpose_reads"] and p["vec_elems"] == 16 and (p["tile_a"], p["tile_b"]) == (16 * ta, 16 * tb), shape
    p = lr.copy_plan(*u8, tuning={"transpose_reads": 1, "pipeline_tiles": 3, "tile_shape": 0})
    assert p["transpose_reads"] and p["pipeline_tiles"] == 3 and p["vec_elems"] == 16
    # chunk_bytes: 16-byte chunks through registers; 8 turns the transpose reads off
    p = lr.copy_plan(*u8, tuning={"chunk_bytes": 16})
    assert p["vec_elems"] == 16 and not p["transpose_reads"] and not p["direct"]
    p = lr.copy_plan(*u8, tuning={"chunk_bytes": 8, "transpose_reads": 1, "direct_loads": 1})
    assert p["vec_elems"] == 8 and not p["transpose_reads"]
    # a layout without 16-byte chunks keeps narrower ones
    odd = ("(4096,4104):(4104,1)", 4096 * 4104, "(4096,4104):(1,4096)", 4096 * 4104, 1)
    assert lr.copy_plan(*odd, tuning={"chunk_bytes": 16})["vec_elems"] == 8


def _table_cycles(words):
    """Cycles of one 32-lane phase reading 4-byte words, per the gfx950 read model
    (32 banks of 4 bytes; a bank serves its distinct words one per cycle)."""
    per_bank = {}
    for wd in set(words):
        per_bank[wd % 32] = per_bank.get(wd % 32, 0) + 1
    return max(per_bank.values())


def test_staged_gather_grouping_is_conflict_free_on_padded_tiles():
    """The padded tiles' gather: with 32 lanes over two tiles (16 chunks each) every
    LDS read is 2-way conflicted in the gfx950 model -- the two tiles' footprints put
    3 words in some banks, and no tile stride evens that out.  Over four tiles x 8
    chunks (one half of each) every read is conflict-free; the planner picks that."""
    w = W.full("padtiles")
    p = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 4)
    assert p["path"] == "staged" and p["gather_chunks"] == 8, p
    # The lane grouping rebuilt here: footprint word of element x of dst chunk c of a
    # tile is 18x + c%8 + 9(c//8), tiles 72 words apart, 32-lane slices of cps chunks
    # from each of 32/cps tiles.  A wave's read of one x is costed phase by phase in
    # the gfx950 read model (4-byte accesses: 32 banks, 32 lanes a phase -- the model
    # tests/test_gpu_lds_model.py holds against the bank-conflict counter).
    def cycles(cps, cpt=16):
        slices, G = cpt // cps, 32 // cps
        total = 0
        for w0 in range(0, 256, 64):
            for x in range(4):
                words = []
                for l in range(64):
                    q, li = (w0 + l) // 32, (w0 + l) % 32
                    kk, c = (q // slices) * G + li // cps, (q % slices) * cps + li % cps
                    words.append(72 * kk + 18 * x + c % 8 + 9 * (c // 8))
                total += sum(_table_cycles(words[h:h + 32]) for h in (0, 32))
        return total
    assert cycles(16) == 2 * cycles(8)       # the old grouping: every phase 2-way
    assert cycles(8) == 4 * 4 * 2            # 4 waves x 4 reads x 2 phases, 1 cycle each
    # the override reproduces the old grouping
    q = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 4, tuning={"gather_chunks": 16})
    assert q["gather_chunks"] == 16
    # a small footprint that is conflict-free either way keeps the widest grouping
    p = lr.copy_plan("((4,8),2,64):((8,1),32,64)", 64 * 64, "((4,8),2,64):((1,4),32,64)", 64 * 64, 4)
    if p["path"] == "staged":
        assert p["gather_chunks"] in (8, 16)


def test_vector_blocked_order_on_the_retile():
    """Traversal order 2 of the vector path: lanes of a wave along the source (8
    tiles' 128-byte rows of one source row), the 4 waves of a workgroup along the
    destination (4 consecutive tile rows), the rest in source order -- the same copy,
    as joint modes split at the wave and workgroup boundaries."""
    w = W.full("retile")
    args = (w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    p = lr.copy_plan(*args, tuning={"vector_order": 2})
    assert p["path"] == "vector" and p["vector_order"] == 2
    assert p["joint"] == [(64, 1, 1), (8, 64, 8192), (4, 4096, 64), (8, 512, 65536), (32, 16384, 256),
                          (32, 524288, 524288)], p["joint"]
    src_order = lr.copy_plan(*args, tuning={"vector_order": 1})["joint"]
    assert src_order == [(64, 1, 1), (64, 64, 8192), (128, 4096, 64), (32, 524288, 524288)], src_order
    # every order covers the same (extent, source, destination) points
    for t in (0, 1, 2):
        j = lr.copy_plan(*args, tuning={"vector_order": t})["joint"]
        assert math.prod(e for e, _, _ in j) == 1 << 24


def test_plan_few_channel_images():
    """NHWC <-> NCHW with 2..8 channels of at most 16 bytes: the channel shuffle (the
    de-interleave one way; the interleave, through LDS unless the channel count is a
    power of two, the other).  Pixel counts that are not a multiple of one 16-byte
    chunk take its element-granular form; swizzles keep the general kernels."""
    def image(n, h, w, c):
        hw = h * w
        return f"({n},{h},{w},{c}):({hw * c},{w * c},{c},1)", f"({n},{h},{w},{c}):({hw * c},{w},1,{hw})"

    for eb in (1, 2, 4, 8):
        for c in range(2, 9):
            nhwc, nchw = image(8, 32, 32, c)
            size = 8 * 32 * 32 * c
            p, q = lr.copy_plan(nhwc, size, nchw, size, eb), lr.copy_plan(nchw, size, nhwc, size, eb)
            if c * eb <= 16:
                assert p["path"] == "deinterleave" and p["tile_a"] == 256 * 16 // eb and p["tile_b"] == c, (eb, c, p)
                assert q["path"] == "interleave", (eb, c, q)
                assert (q["tile_a"] == 256 * 16 // eb) == bool(c & (c - 1)), (eb, c, q)
            else:
                assert p["path"] != "deinterleave"
    # 323 pixels: no whole 16-byte chunks per plane, so the element-granular form
    # (16/eb pixels per lane), for any channel count; a buffer that is not element-
    # aligned keeps the generic kernel
    for c in (3, 4):
        nhwc, nchw = image(3, 17, 19, c)
        for eb in (1, 2, 4):
            for ts, td, path in ((nhwc, nchw, "deinterleave"), (nchw, nhwc, "interleave")):
                p = lr.copy_plan(ts, 3 * 323 * c, td, 3 * 323 * c, eb)
                want = (path, 1, 256 * 16 // eb, -(-323 // (256 * 16 // eb)) * 3) if c * eb <= 16 else ("generic",)
                assert (p["path"], p["vec_elems"], p["tile_a"], p["grid"])[:len(want)] == want, (c, eb, p)
        p = lr.copy_plan(nhwc, 3 * 323 * c, nchw, 3 * 323 * c, 2, src_align=1)
        assert p["path"] == "generic", p
    # its streaming threshold is the 256 MiB last-level cache (its ranges start
    # unaligned, so partial lines merge in the cache below that); aligned planes
    # stream from 64 MiB like the other kernels
    for n, want in ((128, False), (300, True)):
        nhwc, nchw = image(n, 299, 299, 3)
        p = lr.copy_plan(nhwc, n * 89401 * 3, nchw, n * 89401 * 3, 2)
        assert (p["path"], p["vec_elems"], p["streaming"]) == ("deinterleave", 1, want), (n, p)
    nhwc, nchw = image(128, 224, 224, 3)
    p = lr.copy_plan(nhwc, 128 * 50176 * 3, nchw, 128 * 50176 * 3, 2)
    assert (p["path"], p["vec_elems"], p["streaming"]) == ("deinterleave", 8, True), p
    # under one pixel per lane (63 pixels) it is not worth a workgroup of 4096
    nhwc, nchw = image(3, 7, 9, 3)
    assert lr.copy_plan(nhwc, 567, nchw, 567, 2)["path"] == "generic"
    # nor does it take layouts a better kernel handles (the padded tiles look like
    # eight pixels of four channels)
    w = W.full("padtiles")
    assert lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 4)["path"] == "staged"
    assert lr.copy_plan("Sw<1,3,4> o (64,3):(3,1)", 192, "(64,3):(1,64)", 192, 2)["path"] != "deinterleave"
    with pytest.raises(lr.LayoutRemapError):
        lr.copy_plan("(8,8):(1,8)", 64, "(8,8):(1,8)", 64, 2, lr.COPY_FORCE_PATH(lr.PATH_DEINTERLEAVE))


def test_plan_element_tiles_where_chunks_do_not_fit():
    """Transposes whose rows allow no aligned 16-byte chunks take element tiles of
    256-byte rows, except 1-byte elements that still fit 4- or 8-byte chunks; with
    at least as many a-tiles as b-tiles the tiles go a fastest."""
    # (n, bytes per element) -> element tiles?  (8190, 8) and (8192, 2) have full
    # 16-byte chunks; 1-byte elements in 4- and 8-byte chunks keep the chunks
    want = {(8191, 1): True, (8191, 2): True, (8191, 4): True, (8191, 8): True,
            (8190, 1): True, (8188, 1): False, (8184, 1): False, (8190, 2): True, (8190, 4): True,
            (8190, 8): False, (8200, 1): False, (8192, 2): False}
    for (n, eb), element in want.items():
        p = lr.copy_plan(f"({n},{n}):({n},1)", n * n, f"({n},{n}):(1,{n})", n * n, eb)
        assert p["path"] == "transpose"
        got = p["vec_elems"] == 1 and p["tile_a"] == p["tile_b"] == 256 // eb and p["block"] == 512
        assert got == element, (n, eb, p)
        if element:  # as many a-tiles as b-tiles: a fastest; ordinary accesses at any size
            assert p["order"] == 0 and not p["streaming"], (n, eb, p)
    for r, c, order in ((4097, 16383, 0), (16383, 4097, 1)):
        p = lr.copy_plan(f"({r},{c}):({c},1)", r * c, f"({r},{c}):(1,{r})", r * c, 1)
        assert p["tile_a"] == 256 and p["order"] == order, (r, c, p)
    p = lr.copy_plan("(8188,8188):(8188,1)", 8188 ** 2, "(8188,8188):(1,8188)", 8188 ** 2, 1,
                     tuning={"element_tiles": 1})
    assert p["tile_a"] == 256
    p = lr.copy_plan("(8191,8191):(8191,1)", 8191 ** 2, "(8191,8191):(1,8191)", 8191 ** 2, 2,
                     tuning={"element_tiles": 0})
    assert p["tile_a"] == 16


def test_plan_errors():
    E = lr.binding
    with pytest.raises(lr.LayoutRemapError) as e:
        lr.copy_plan("8:1", 8, "4:1", 4, 4)
    assert e.value.code == E.ERR_SIZE_MISMATCH
    with pytest.raises(lr.LayoutRemapError) as e:
        lr.copy_plan("8:1", 7, "8:1", 8, 4)
    assert e.value.code == E.ERR_BOUNDS
    with pytest.raises(lr.LayoutRemapError) as e:
        lr.copy_plan("(8,8):(1,8)", 64, "((4,2),(2,4)):((2,16),(1,8))", 64, 4)
    assert e.value.code == E.ERR_ALIAS
    with pytest.raises(lr.LayoutRemapError) as e:
        lr.copy_plan("8:1", 8, "8:1", 8, 3)
    assert e.value.code == E.ERR_ELEM_BYTES
    with pytest.raises(lr.LayoutRemapError) as e:
        lr.copy_plan("8:1", 8, "8:1", 8, 4, lr.COPY_FORCE_PATH(lr.PATH_TRANSPOSE))
    assert e.value.code == E.ERR_PATH
    with pytest.raises(lr.LayoutRemapError) as e:  # ordered alias beyond its limits
        lr.copy_plan("(67108864,2):(1,67108864)", 1 << 27, "(67108864,2):(1,0)", 1 << 26, 1,
                     lr.COPY_ORDERED_ALIAS)
    assert e.value.code == E.ERR_ALIAS
    with pytest.raises(lr.LayoutRemapError) as e:  # destination cosize above 2^26
        lr.copy_plan("(134217728,2):(1,134217728)", 1 << 28, "(134217728,2):(1,0)", 1 << 27, 1,
                     lr.COPY_ORDERED_ALIAS)
    assert e.value.code == E.ERR_ALIAS
    p = lr.copy_plan("(1048576,128):(1,1048576)", 1 << 27, "(1048576,128):(1,0)", 1 << 20, 1, lr.COPY_ORDERED_ALIAS)
    assert p["path"] == "alias" and p["grid"] == 128
    p = lr.copy_plan("(8,8):(1,8)", 64, "((4,2),(2,4)):((2,16),(1,8))", 64, 4, lr.COPY_ORDERED_ALIAS)
    assert p["path"] == "alias" and p["grid"] == 1


def test_plan_alignment_drops_vector_width():
    w = W.full("retile")
    for align, want in [(16, 8), (8, 4), (4, 2), (2, 1)]:
        p = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2, src_align=align)
        assert p["vec_elems"] == want, align


def test_plan_wide_index_for_big_offsets():
    # offsets beyond 32 bits: four blocks (one per far source row) at offset bases,
    # or one 64-bit launch when asked for
    p = lr.copy_plan("(2,4):(1,1099511627776)", 3298534883330, "(2,4):(4,1)", 8, 1)
    assert not p["wide"] and p["blocks"] == 4 and p["path"] == "generic"
    p = lr.copy_plan("(2,4):(1,1099511627776)", 3298534883330, "(2,4):(4,1)", 8, 1, lr.COPY_WIDE_INDEX)
    assert p["wide"] and p["blocks"] == 1 and p["path"] == "generic"
    p = lr.copy_plan("64:1", 64, "64:1", 64, 4, lr.COPY_WIDE_INDEX)
    assert p["wide"] and p["path"] == "vector" and p["vec_elems"] == 4
    # more than 2^31 elements: 64-bit indices, still 16-byte vectors along a common
    # contiguous mode; a forced generic plan moves single elements
    n = (1 << 31) + 16
    p = lr.copy_plan(f"{n}:1", n, f"{n}:1", n, 1, lr.COPY_WIDE_INDEX)
    assert p["wide"] and p["path"] == "vector" and p["vec_elems"] == 16 and p["grid"] == -(-n // 16 // 1024)
    assert p["blocks"] == 1
    p = lr.copy_plan(f"{n}:1", n, f"{n}:1", n, 1, lr.COPY_FORCE_PATH(lr.PATH_GENERIC))
    assert p["path"] == "generic" and p["vec_elems"] == 1 and p["wide"] and p["blocks"] == 1
    # by default such a copy is cut into blocks that each fit 32-bit offsets
    p = lr.copy_plan(f"{n}:1", n, f"{n}:1", n, 1)
    assert p["blocks"] == 2 and not p["wide"] and p["path"] == "vector" and p["n_elems"] == n
    # a 65536^2 fp16 transpose: four 32768^2 blocks on the transpose path
    m = 65536
    p = lr.copy_plan(f"({m},{m}):({m},1)", m * m, f"({m},{m}):(1,{m})", m * m, 2)
    assert p["blocks"] == 4 and not p["wide"] and p["path"] == "transpose" and p["streaming"]
    assert p["grid"] == (32768 // 256) ** 2
    # a swizzle keeps the single 64-bit launch
    p = lr.copy_plan(f"Sw<3,3,3> o ({m},{m}):({m},1)", m * m, f"({m},{m}):(1,{m})", m * m, 2)
    assert p["blocks"] == 1 and p["wide"]
    p = lr.copy_plan("(16,3):(1,32)", 96, "(16,3):(1,16)", 48, 2, lr.COPY_WIDE_INDEX)
    assert p["path"] == "vector" and p["vec_elems"] == 8
    with pytest.raises(lr.LayoutRemapError):
        lr.copy_plan("(8,8):(8,1)", 64, "(8,8):(1,8)", 64, 2, lr.COPY_WIDE_INDEX | lr.COPY_FORCE_PATH(lr.PATH_TRANSPOSE))


# ---------------------------------------------------------------------------
# Multiply-high division constants: built with g++ from the library's own host
# sources, checked exhaustively for a few divisors over all 31-bit dividends and
# at every quotient boundary for many more.  Also run under ASan/UBSan with a
# random walk through the host algebra.
# ---------------------------------------------------------------------------
def _gpp(tmp_path, sanitize=False):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    exe = str(tmp_path / ("host_check_san" if sanitize else "host_check"))
    src = [os.path.join(ROOT, "tests", "host_check.cpp"),
           os.path.join(ROOT, "layout_remapping_copy_amd", "csrc", "host_layout.cpp"),
           os.path.join(ROOT, "layout_remapping_copy_amd", "csrc", "inspect.cpp"),
           os.path.join(ROOT, "layout_remapping_copy_amd", "csrc", "plan.cpp")]
    flags = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"] if sanitize else ["-O2"]
    cmd = ["g++", "-std=c++17", *flags, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "layout_remapping_copy_amd", "csrc"), *src, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    return exe


def test_fastdiv_exact(tmp_path):
    exe = _gpp(tmp_path)
    r = subprocess.run([exe, "fastdiv"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "fastdiv ok" in r.stdout


def test_host_algebra_under_sanitizers(tmp_path):
    exe = _gpp(tmp_path, sanitize=True)
    r = subprocess.run([exe, "fuzz"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "fuzz ok" in r.stdout


def test_batched_plan():
    """The batched path: whole compact small matrices per wavefront.  The planner takes
    it for 2-byte elements (up to 8 KiB a matrix), and for other small matrices the
    staged path does not take; it keeps the staged path for 4- and 8-byte elements
    and the transpose for their 8 KiB matrices.  The LDS swizzle is conflict-free in the
    bank model for power-of-two matrices and is an involution inside 16-chunk groups."""
    def bt(A, B, n, eb):
        return (f"({B},{A},{n}):({A},1,{A * B})", A * B * n, f"({B},{A},{n}):(1,{B},{A * B})", A * B * n, eb)
    assert lr.copy_plan(*bt(16, 16, 4096, 2))["path"] == "batched"
    assert lr.copy_plan(*bt(32, 32, 4096, 2))["path"] == "batched"
    assert lr.copy_plan(*bt(24, 24, 4096, 2))["path"] == "batched"
    assert lr.copy_plan(*bt(16, 16, 4096, 4))["path"] == "staged"
    assert lr.copy_plan(*bt(16, 16, 4096, 8))["path"] == "staged"
    assert lr.copy_plan(*bt(64, 64, 4096, 2))["path"] == "batched"
    assert lr.copy_plan(*bt(64, 32, 4096, 4))["path"] == "transpose"
    force = lr.COPY_FORCE_PATH(lr.PATH_BATCHED)
    for A, B, eb in ((16, 16, 2), (32, 32, 2), (64, 64, 2), (16, 32, 2), (8, 16, 2), (8, 8, 4), (16, 16, 4),
                     (32, 64, 4), (4, 4, 8), (16, 16, 8), (32, 32, 8)):
        p = lr.copy_plan(*bt(A, B, 1000, eb), flags=force)
        V = 16 // eb
        cpm = A * B // V
        assert p["path"] == "batched" and p["block"] == 64 and p["batch_matrices"] == 512 // cpm
        assert p["grid"] == -(-1000 // p["batch_matrices"]) and (p["tile_a"], p["tile_b"]) == (A, B)
        s0, m0, t0, s1, m1, t1 = p["batch_swizzle"]

        def swz(c):
            return c ^ (((c >> s0) & m0) << t0) ^ (((c >> s1) & m1) << t1)
        assert all(swz(swz(c)) == c and swz(c) >> 4 == c >> 4 for c in range(1024))
        # the gfx950 model: 16-byte reads in phases of 16 lanes over 64 banks, writes in
        # phases of 8 over 32; every phase of both exchanges touches distinct bank groups
        P, Q = A // V, B // V
        nblk = p["batch_matrices"] * P * Q
        for r in range(0, nblk, 64):
            lanes = []
            for u in range(r, min(nblk, r + 64)):
                mi, rest = divmod(u, P * Q)
                ba, bb = (rest // Q, rest % Q) if p["batch_order"] else (rest % P, rest // P)
                lanes.append((mi, ba, bb))
            for j in range(V):
                rd = [swz(mi * cpm + (V * bb + j) * P + ba) for mi, ba, bb in lanes]
                wr = [swz(mi * cpm + (V * ba + j) * Q + bb) for mi, ba, bb in lanes]
                for q in range(0, len(rd), 16):
                    assert len({x % 16 for x in rd[q:q + 16]}) == len(rd[q:q + 16]), (A, B, eb, "read")
                for q in range(0, len(wr), 8):
                    assert len({x % 8 for x in wr[q:q + 8]}) == len(wr[q:q + 8]), (A, B, eb, "write")
    # not compact, too large, or narrow chunks: the path does not apply
    for args in (("(16,16,64):(17,1,272)", 272 * 64, "(16,16,64):(1,16,256)", 256 * 64, 2),
                 ("(128,64,8):(64,1,8192)", 8192 * 8, "(128,64,8):(1,128,8192)", 8192 * 8, 2),
                 ("(12,12,64):(12,1,144)", 144 * 64, "(12,12,64):(1,12,144)", 144 * 64, 2)):
        with pytest.raises(lr.LayoutRemapError):
            lr.copy_plan(*args, flags=force)


def test_plan_cache_returns_the_same_plans():
    """Plans are cached per thread by their full input: asking again gives the same
    plan (or the same error), and any change of input (capacity, alignment, tuning,
    flags, a stride) gives that input's own plan."""
    w = W.full("transpose")
    args = (w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    first = lr.copy_plan(*args)
    for _ in range(3):
        assert lr.copy_plan(*args) == first
    t = lr.copy_plan(*args, tuning={"tile_shape": 1})
    assert t["tile_b"] != first["tile_b"] and lr.copy_plan(*args) == first
    assert lr.copy_plan(*args, tuning={"tile_shape": 1}) == t
    odd = lr.copy_plan(*args, src_align=2)
    assert odd != first and lr.copy_plan(*args, src_align=2) == odd
    assert lr.copy_plan(*args, src_align=48) == first  # 48 = 16 * 3: aligned to 16
    for _ in range(2):
        with pytest.raises(lr.LayoutRemapError) as e:
            lr.copy_plan(*args, flags=lr.COPY_FORCE_PATH(lr.PATH_INTERLEAVE))
        assert e.value.code == lr.binding.ERR_PATH
    other = lr.copy_plan("(8192,8192):(8193,1)", 8192 * 8193, w.dst_layout, w.dst_elems, 2)
    assert other["joint"] != first["joint"]
    # more distinct inputs than the cache holds, then the first again
    for k in range(40):
        lr.copy_plan(f"({64 + k},64):(64,1)", (64 + k) * 64, f"({64 + k},64):(1,{64 + k})", (64 + k) * 64, 4)
    assert lr.copy_plan(*args) == first


def test_workgroup_lanes_plan():
    """workgroup_lanes: 64, 128 or 256 lanes per workgroup on the vector/generic kernel with
    one unit per lane and on the narrow interleave; the grid (and the interleave's tile)
    follow; tiles of atoms and 64-bit copies keep 256.  The planner takes one wavefront
    for the interleave and single contiguous runs from a 64 MiB footprint."""
    w = W.full("interleave")
    args = (w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    base = lr.copy_plan(*args)
    for lanes in (64, 128, 256):
        p = lr.copy_plan(*args, tuning={"workgroup_lanes": lanes})
        assert p["path"] == "interleave" and p["block"] == lanes
        assert p["tile_a"] * base["block"] == base["tile_a"] * lanes and p["grid"] * lanes == base["grid"] * base["block"]
    n = 3 * (1 << 20) + 77
    for lanes in (64, 128):
        p = lr.copy_plan(f"{n}:1", n, f"{n}:1", n, 16, tuning={"workgroup_lanes": lanes})
        assert p["path"] in ("vector", "generic") and p["block"] == lanes and p["grid"] == -(-n // lanes)
    r = W.full("retile")
    p = lr.copy_plan(r.src_layout, r.src_elems, r.dst_layout, r.dst_elems, 2, tuning={"workgroup_lanes": 64})
    assert p["vector_order"] == 3 and p["block"] == 64
    p = lr.copy_plan(f"{n}:1", n, f"{n}:1", n, 16, flags=lr.COPY_WIDE_INDEX, tuning={"workgroup_lanes": 64})
    assert p["wide"] and p["block"] == 256
    assert base["block"] == 64 and lr.copy_plan(f"{n}:1", n, f"{n}:1", n, 16)["block"] == 64  # 96 MiB moved
    small = 1 << 19  # 16 MiB moved
    assert lr.copy_plan(f"{small}:1", small, f"{small}:1", small, 16)["block"] == 256
    s = W.small("interleave")
    assert lr.copy_plan(s.src_layout, s.src_elems, s.dst_layout, s.dst_elems, 2)["block"] == 256
    perm = ("(2048,1024,64):(1,2048,2097152)", 1 << 27, "(2048,1024,64):(1,131072,2048)", 1 << 27, 2)
    assert lr.copy_plan(*perm)["block"] == 256  # three modes
    # the staged gather: two destination chunks a lane, so tiles a workgroup scale with lanes,
    # and at least one lane per destination chunk of a tile (2 KiB rows: 128 chunks)
    pt = W.full("padtiles")
    pargs = (pt.src_layout, pt.src_elems, pt.dst_layout, pt.dst_elems, 4)
    pbase = lr.copy_plan(*pargs)
    for lanes in (64, 128, 256):
        p = lr.copy_plan(*pargs, tuning={"workgroup_lanes": lanes})
        assert p["path"] == "staged" and p["block"] == lanes
        assert p["tile_a"] * pbase["block"] == pbase["tile_a"] * lanes and p["grid"] * lanes == pbase["grid"] * pbase["block"]
    rows = ("(512,30):(1,520)", 520 * 30, "(512,30):(1,512)", 512 * 30, 4)
    p = lr.copy_plan(*rows, flags=lr.COPY_FORCE_PATH(lr.PATH_STAGED), tuning={"workgroup_lanes": 64})
    assert p["block"] == 128 and p["tile_a"] == 2 and p["gather_chunks"] == 32
