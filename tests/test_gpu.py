"""GPU parity: the HIP path through the C ABI against the CPU oracle, byte for byte.

Every destination buffer starts filled with 0xA5 and is compared whole, so
positions a layout does not reach are checked to stay untouched.  Full-size
workloads run in the same launch configuration as bench.py and are compared
whole against NumPy closed forms (each pinned to the oracle's copy) and at
sampled indices against the oracle's own evaluation.
"""

import os
import random
import sys

import numpy as np
import pytest

import oracle as O
from oracle import forms as F
import workloads as W

torch = pytest.importorskip("torch")
import layout_remapping_copy_amd as lr  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(lr.LIB_PATH), "liblayout_remap.so is not built"
    lr.lib()
    return torch.device("cuda:0")


class Knobs:
    """Overrides of the planner's launch choices (lr_copy_tuning fields) that every
    copy and plan call of this module passes while a test holds them."""

    def __init__(self):
        self.t = {}

    def set(self, **kw):
        self.t.update(kw)

    def unset(self, *names):
        for n in names:
            self.t.pop(n, None)

    def policy(self, nt, sc1=None):
        """nt "0": ordinary loads and stores; "1": non-temporal, the stores with the
        sc1 bit where the kernel has buffer stores unless sc1 is "0"."""
        self.unset("load_policy", "store_policy")
        if nt == "0":
            self.set(load_policy=0)
        else:
            self.set(load_policy=2)
            if sc1 == "0":
                self.set(store_policy=2)

    def tuning(self):
        return dict(self.t) or None


KNOBS = Knobs()


@pytest.fixture
def knobs():
    KNOBS.t.clear()
    yield KNOBS
    KNOBS.t.clear()


def plan(Ls, ns, Ld, nd, eb, flags=0, **kw):
    return lr.copy_plan(Ls, ns, Ld, nd, eb, flags, tuning=KNOBS.tuning(), **kw)


def copy_(s, Ls, d, Ld, elem_bytes, flags=0):
    return lr.layout_copy(s, Ls, d, Ld, elem_bytes=elem_bytes, flags=flags, tuning=KNOBS.tuning())


def gpu_copy(dev, src, Ls, dst, Ld, eb, flags=0, src_off=0, dst_off=0):
    s = torch.zeros(src.nbytes + src_off, dtype=torch.uint8, device=dev)
    d = torch.zeros(dst.nbytes + dst_off, dtype=torch.uint8, device=dev)
    s[src_off:] = torch.from_numpy(src).to(dev)
    d[dst_off:] = torch.from_numpy(dst).to(dev)
    copy_(s[src_off:], Ls, d[dst_off:], Ld, eb, flags)
    torch.cuda.synchronize()
    return d[dst_off:].cpu().numpy()


def gpu_eval(dev, L, n=None, idx=None):
    t = lr.layout_eval(L, idx=idx, n=n, device=dev)
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ---------------------------------------------------------------------------
# Evaluation
# ---------------------------------------------------------------------------
EVAL_LAYOUTS = ["((4,8),2):((16,1),8)", "Sw<3,0,3> o (8,8):(8,1)", "((4,2),(2,4)):((2,16),(1,8))", "(4,2):(2,1)",
                "(4,2):(1,4)", "(4,2,2):(8,2,1)", "Sw<3,3,3> o ((128,32),(64,64)):((64,524288),(1,8192))",
                "(8,4,2):(1,16,512)", "(8,2):(1,16)", "((4,8),2,1000):((18,1),9,72)"]


@pytest.mark.parametrize("text", EVAL_LAYOUTS)
def test_eval_layouts(dev, text):
    say("eval", text)
    L = O.parse(text)
    got = gpu_eval(dev, text)
    want = O.eval_indices(L, np.arange(O.size(L)))
    assert np.array_equal(got, want)


def test_eval_thread_maps(dev):
    for p, s, k, t in [(8, 4, 16, 64), (8, 2, 16, 32), (4, 3, 17, 96)]:
        say("eval thread map", p, s, k, t)
        L = lr.thread_map(p, s, k, t)
        got = gpu_eval(dev, L, n=t)
        assert got.tolist() == [O.stripmined_offset(i, p, s, k) for i in range(t)]
        B = lr.thread_map(p, 0, k, t)
        got = gpu_eval(dev, B, n=t)
        assert got.tolist() == [O.pitch_linear_offset(i, p, k) for i in range(t)]


def test_eval_indices_and_out_of_range(dev):
    say("eval idx")
    text = "((4,8),2):((16,1),8)"
    idx = torch.tensor([5, 0, 63, -1, 64, 17, 1 << 40], dtype=torch.int64, device=dev)
    got = gpu_eval(dev, text, idx=idx)
    L = O.parse(text)
    assert got.tolist() == [O.eval_index(L, 5), 0, 63, -1, -1, O.eval_index(L, 17), -1]


def test_eval_coords(dev):
    say("eval coords")
    text = "((4,2),(2,4)):((2,16),(1,8))"
    L = O.parse(text)
    rc = [(r, c) for r in range(8) for c in range(8)] + [(8, 0), (0, -1)]
    t = torch.tensor(rc, dtype=torch.int64, device=dev)
    got = lr.layout_eval_coords(text, t).cpu().tolist()
    assert got[:64] == [O.eval_coord(L, x) for x in rc[:64]] and got[64:] == [-1, -1]
    nat = [(i0, i1, j0, j1) for i0 in range(4) for i1 in range(2) for j0 in range(2) for j1 in range(4)]
    t = torch.tensor(nat + [(4, 0, 0, 0)], dtype=torch.int64, device=dev)
    got = lr.layout_eval_coords(text, t).cpu().tolist()
    assert got[:-1] == [O.eval_coord(L, ((a, b), (c, d))) for a, b, c, d in nat] and got[-1] == -1
    # golden: blocked natural coordinates and the swizzle
    assert got[nat.index((0, 1, 0, 0))] == 16 and got[nat.index((1, 0, 0, 0))] == 2
    sw = torch.tensor([(2, 0), (2, 1)], dtype=torch.int64, device=dev)
    assert lr.layout_eval_coords("Sw<3,0,3> o (8,8):(8,1)", sw).cpu().tolist() == [18, 19]


def test_eval_coords_random(dev):
    """Per-mode coordinates of random nested layouts (32-bit and 64-bit offset
    ranges), in range and out of range, against the oracle."""
    rng = random.Random(37)
    for i in range(60):
        nm = rng.randint(1, 4)
        modes = []
        for _ in range(nm):
            nl = rng.randint(1, 3)
            ext = [rng.randint(1, 6) for _ in range(nl)]
            big = i % 3 == 0
            st = [rng.randint(0, 40) * (1 << 29 if big else 1) for _ in range(nl)]
            if nl == 1:
                modes.append((f"{ext[0]}", f"{st[0]}"))
            else:
                modes.append(("(" + ",".join(map(str, ext)) + ")", "(" + ",".join(map(str, st)) + ")"))
        t = "(" + ",".join(m[0] for m in modes) + "):(" + ",".join(m[1] for m in modes) + ")"
        L = O.parse(t)
        sizes = [O.size(O.parse(f"{m[0]}:{m[1]}")) for m in modes]
        rows = [tuple(rng.randint(0, sz - 1) for sz in sizes) for _ in range(40)]
        rows += [tuple(sz if j == 0 else 0 for j, sz in enumerate(sizes)), tuple(-1 for _ in sizes)]
        ct = torch.tensor(rows, dtype=torch.int64, device=dev)
        got = lr.layout_eval_coords(t, ct).cpu().tolist()
        want = [O.eval_coord(L, r) for r in rows[:-2]] + [-1, -1]
        assert got == want, (t, rows[:3])


def _rand_text(rng, swz=True, max_leaves=5):
    nl = rng.randint(1, max_leaves)
    ext = [rng.randint(1, 7) for _ in range(nl)]
    st = [rng.randint(0, 50) for _ in range(nl)]
    t = "(" + ",".join(map(str, ext)) + "):(" + ",".join(map(str, st)) + ")"
    if swz and rng.random() < 0.3:
        b = rng.randint(1, 3)
        t = f"Sw<{b},{rng.randint(0, 3)},{rng.randint(b, 4)}> o " + t
    return t


def test_eval_random(dev):
    rng = random.Random(31)
    for i in range(200):
        t = _rand_text(rng)
        if i % 50 == 0:
            say("eval random", i, t)
        L = O.parse(t)
        assert np.array_equal(gpu_eval(dev, t), O.eval_indices(L, np.arange(O.size(L)))), t


def test_eval_ranges_pairwise(dev):
    """Index ranges of layouts whose offsets fit 31 bits run two indices per lane (the
    second by a step of leaf 0 when its digit does not wrap) with 16-byte stores:
    odd counts, counts past the size (-1 there), leaf-0 extents of 1 and 2,
    swizzles, and an output only 8-byte aligned (one index per lane)."""
    import ctypes
    texts = ["Sw<3,3,3> o ((128,32),(64,64)):((64,524288),(1,8192))", "(1,7,3):(5,1,7)", "(2,9,5):(90,10,1)",
             "((4,8),2,(3,5)):((16,1),8,(64,192))", "Sw<2,1,3> o (3,5,7):(35,7,1)", "5:0", "2147483:1000", "2147484:1001"]
    for t in texts:
        L = O.parse(t)
        size = O.size(L)
        for n in sorted({1, 2, 5, size, size + 3}):
            ks = np.arange(n)
            want = np.where(ks < size, O.eval_indices(L, np.minimum(ks, size - 1)), -1)
            say("eval range", t, "n", n)
            assert np.array_equal(gpu_eval(dev, t, n=n), want), (t, n)
            # an output starting 8 bytes into an allocation
            buf = torch.full((n + 1,), 7, dtype=torch.int64, device=dev)
            Lc = lr.parse(t)
            rc = lr.binding.lib().lr_layout_eval(ctypes.byref(Lc.c), None, n, ctypes.c_void_p(buf.data_ptr() + 8),
                                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert rc == 0
            torch.cuda.synchronize()
            got = buf.cpu().numpy()
            assert got[0] == 7 and np.array_equal(got[1:], want), (t, n)


def test_eval_wide(dev):
    say("eval wide")
    text = "(65536,65536):(65536,1)"  # 2^32 indices: 64-bit division path
    L = O.parse(text)
    ks = np.random.default_rng(5).integers(0, 1 << 32, 100000, dtype=np.int64)
    got = gpu_eval(dev, text, idx=torch.from_numpy(ks).to(dev))
    assert np.array_equal(got, O.eval_indices(L, ks))


# ---------------------------------------------------------------------------
# Copies at sizes the oracle finishes quickly
# ---------------------------------------------------------------------------
def test_algebra_built_layouts_on_device(dev):
    """Layouts built by the library's algebra -- slice of a zipped_divide,
    (A, complement(A)), logical_divide, blocked_product -- evaluated and used as
    copy layouts on the GPU, byte-exact against the oracle's own construction of
    the same layouts ([CuTe algebra page, sections 3.2 and 4.1])."""
    rng = np.random.default_rng(17)
    cases = []
    # tile (3,5) of the 128 x 128 column-major matrix split by 4 x 8
    Z = lr.zipped_divide("(128,128):(1,128)", (4, 8))
    T, off = lr.slice(Z, (-1, 3 + 32 * 5))
    To, offo = O.slice_layout(O.zipped_divide(O.parse("(128,128):(1,128)"), (4, 8)), (None, (3, 5)))
    assert off == offo == 5132
    cases.append(("slice tile (3,5)", T, To, off))
    # every tile of a 1024 x 512 matrix in 64 x 32 tiles: the same slice per tile
    Zb = lr.zipped_divide("(1024,512):(512,1)", (64, 32))
    Tb, offb = lr.slice(Zb, (-1, 7 + 16 * 9))
    Tbo, offbo = O.slice_layout(O.zipped_divide(O.parse("(1024,512):(512,1)"), (64, 32)), (None, 7 + 16 * 9))
    assert offb == offbo
    cases.append(("slice tile (7,9) of 1024x512", Tb, Tbo, offb))
    # a tile and what it leaves over: (A, complement(A, M)) is a bijection onto [0, M)
    A = "(4,8):(1,16)"
    C = lr.complement(A, 2048)
    Co = O.complement(O.parse(A), 2048)
    assert C.leaves == O.flatten(Co)
    AC = lr.parse(f"(({A.split(':')[0][1:-1]}),({','.join(str(n) for n, _ in C.leaves)})):"
                  f"(({A.split(':')[1][1:-1]}),({','.join(str(d) for _, d in C.leaves)}))")
    ACo = O.parse(str(AC))
    assert sorted(O.eval_indices(ACo, np.arange(O.size(ACo))).tolist()) == list(range(2048))
    cases.append(("(A, complement(A, 2048))", AC, ACo, 0))
    # logical_divide of a 4096-element run by 8:4 (tiles of 8 elements 4 apart)
    D = lr.logical_divide("4096:1", "8:4")
    Do = O.logical_divide(O.parse("4096:1"), O.parse("8:4"))
    assert D.leaves == O.flatten(Do)
    cases.append(("logical_divide(4096:1, 8:4)", D, Do, 0))
    # [CuTe algebra page, section 4.1]: a 4 x 8 block over a 2 x 5 grid, and a
    # 16 x 64 block over a 32 x 16 grid (a 512 x 1024 blocked matrix)
    for a, b in (("(4,8):(1,4)", "(2,5):(1,2)"), ("(16,64):(1,16)", "(32,16):(1,32)")):
        Bp = lr.blocked_product(a, b)
        Bpo = O.blocked_product(O.parse(a), O.parse(b))
        assert Bp.leaves == O.flatten(Bpo)
        cases.append((f"blocked_product({a}, {b})", Bp, Bpo, 0))
    for name, Lc, Lo, base in cases:
        n = O.size(Lo)
        # evaluation of every index on the GPU
        got = gpu_eval(dev, Lc, n=n)
        assert np.array_equal(got, O.eval_indices(Lo, np.arange(n))), name
        for eb in (2, 4):
            cos = O.cosize(Lo) + base
            # gather through the built layout (source at the slice's base offset)
            src = rng.integers(0, 256, cos * eb, dtype=np.uint8)
            dst = np.full(n * eb, 0xA5, np.uint8)
            want = O.copy(src[base * eb:], Lo, dst, O.parse(f"{n}:1"), eb)
            got = gpu_copy(dev, src[base * eb:].copy(), Lc, dst, f"{n}:1", eb)
            say("algebra layouts", name, "gather eb", eb)
            assert np.array_equal(got, want), (name, eb)
            # scatter through it (a bijection onto its image; holes keep 0xA5)
            src2 = rng.integers(0, 256, n * eb, dtype=np.uint8)
            dst2 = np.full((cos - base) * eb, 0xA5, np.uint8)
            want = O.copy(src2, O.parse(f"{n}:1"), dst2, Lo, eb)
            got = gpu_copy(dev, src2, f"{n}:1", dst2, Lc, eb)
            say("algebra layouts", name, "scatter eb", eb)
            assert np.array_equal(got, want), (name, eb)


def _oracle_copy(w):
    src, dst = W.make_src(w), W.make_dst(w)
    want = O.copy(src, O.parse(w.src_layout), dst, O.parse(w.dst_layout), w.elem_bytes,
                  ordered_alias=w.ordered_alias)
    return src, dst, want


@pytest.mark.parametrize("name", list(W.FULL))
def test_copy_small_workloads(dev, name):
    w = W.small(name)
    say("copy small", w.name, w.src_layout, "->", w.dst_layout)
    src, dst, want = _oracle_copy(w)
    flags = lr.COPY_ORDERED_ALIAS if w.ordered_alias else 0
    got = gpu_copy(dev, src, w.src_layout, dst, w.dst_layout, w.elem_bytes, flags)
    assert np.array_equal(got, want)


def test_copy_tile8x8_aliased(dev):
    w = W.tile8x8()
    src, dst, want = _oracle_copy(w)
    say("copy tile8x8 default flags")
    with pytest.raises(lr.LayoutRemapError) as e:
        gpu_copy(dev, src, w.src_layout, dst, w.dst_layout, 4, 0)
    assert e.value.code == lr.binding.ERR_ALIAS
    got = gpu_copy(dev, src, w.src_layout, dst, w.dst_layout, 4, lr.COPY_ORDERED_ALIAS)
    idx = [0, 8, 1, 9, 2, 10, 3, 11, 16, 24, 17, 25, 18, 26, 19, 27, 32, 40, 33, 41, 34, 42, 35, 43,
           48, 56, 49, 57, 50, 58, 51, 59, 36, 44, 37, 45, 38, 46, 39, 47, 52, 60, 53, 61, 54, 62, 55, 63]
    assert got.view(np.uint32)[:48].tolist() == src.view(np.uint32)[idx].tolist()
    assert np.all(got[48 * 4:] == 0xA5)
    assert np.array_equal(got, want)


ALL_PATHS = [lr.PATH_GENERIC, lr.PATH_VECTOR, lr.PATH_TRANSPOSE, lr.PATH_TRANSPOSE_DIRECT, lr.PATH_INTERLEAVE,
             lr.PATH_DEINTERLEAVE, lr.PATH_STAGED, lr.PATH_DUAL, lr.PATH_ALIAS, lr.PATH_BATCHED]


def _case_pairs():
    """Layout pairs (src, dst, src_elems, dst_elems, eb) that admit the various paths."""
    cases = []
    for name in ["transpose", "retile", "interleave", "interleave_cm", "nhwc2nchw", "padtiles"]:
        w = W.small(name)
        cases.append((w.src_layout, w.dst_layout, w.src_elems, w.dst_elems, w.elem_bytes))
    # transposes at every element size, ragged tile edges
    for eb, (r, c) in [(1, (272, 48)), (2, (136, 24)), (4, (40, 36)), (8, (34, 6)), (16, (17, 5)), (2, (7, 9))]:
        cases.append((f"({r},{c}):({c},1)", f"({r},{c}):(1,{r})", r * c, r * c, eb))
    # interleave of a short dst-contiguous mode at every element size
    for eb, nb in [(1, 2), (1, 4), (1, 8), (1, 16), (2, 2), (2, 4), (2, 8), (4, 2), (4, 4), (8, 2)]:
        a, bt = 16 // eb * 6, 3
        cases.append((f"({nb},{a},{bt}):({a},1,{a * nb})", f"({nb},{a},{bt}):(1,{nb},{a * nb})", a * nb * bt,
                      a * nb * bt, eb))
    # padded tiles at two element sizes, swizzled and vector copies
    for eb in (2, 4):
        t = 37
        cases.append((f"((4,8),2,{t}):((18,1),9,72)", f"((4,8),2,{t}):((1,4),32,64)", 72 * t, 64 * t, eb))
    cases.append(("(64,64):(64,1)", "Sw<3,3,3> o (64,64):(64,1)", 4096, 4096, 2))
    cases.append(("Sw<2,2,3> o (32,32):(32,1)", "(32,32):(1,32)", 1024, 1024, 4))
    cases.append(("(96,5,3):(1,96,480)", "(96,5,3):(1,288,96)", 1440, 1440, 2))
    # non-refinable pair (dual) and a broadcast source
    cases.append(("(6,4):(1,6)", "(4,6):(1,4)", 24, 24, 4))
    cases.append(("(8,16):(0,1)", "(8,16):(16,1)", 16, 128, 8))
    return cases


@pytest.mark.parametrize("ci", range(len(_case_pairs())))
def test_copy_every_path(dev, ci):
    ts, td, ns, nd, eb = _case_pairs()[ci]
    rng = np.random.default_rng(ci)
    src = rng.integers(0, 256, ns * eb, dtype=np.uint8)
    dst = np.full(nd * eb, 0xA5, np.uint8)
    want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
    ran = []
    for path in ALL_PATHS:
        flags = lr.COPY_FORCE_PATH(path)
        try:
            plan(ts, ns, td, nd, eb, flags)
        except lr.LayoutRemapError as e:
            assert e.code == lr.binding.ERR_PATH
            continue
        say("copy path", lr.binding.PATH_NAMES[path], ts, "->", td, "eb", eb)
        got = gpu_copy(dev, src, ts, dst, td, eb, flags)
        assert np.array_equal(got, want), lr.binding.PATH_NAMES[path]
        ran.append(path)
    # also the default plan and the 64-bit index variant
    got = gpu_copy(dev, src, ts, dst, td, eb, 0)
    assert np.array_equal(got, want)
    try:
        got = gpu_copy(dev, src, ts, dst, td, eb, lr.COPY_WIDE_INDEX)
        assert np.array_equal(got, want)
    except lr.LayoutRemapError as e:
        assert e.code == lr.binding.ERR_PATH
    assert len(ran) >= 2


def _rand_pair(rng):
    nd = rng.randint(1, 4)
    exts = [rng.choice([1, 2, 3, 4, 5, 7, 8, 16, 24, 32, 40, 64, 72, 100, 128]) for _ in range(nd)]
    while np.prod(exts) > (1 << 17):
        exts[rng.randrange(nd)] = rng.choice([2, 3, 4, 8])

    def compact(order, pad):
        st, w = [0] * nd, 1
        for i in order:
            st[i] = w
            w *= exts[i] + (pad if i == order[0] else 0)
        return st, w

    o1, o2 = list(range(nd)), list(range(nd))
    rng.shuffle(o1)
    rng.shuffle(o2)
    ss, ns = compact(o1, rng.choice([0, 0, 1, 3]))
    sd, nd_ = compact(o2, 0)
    ts = "(" + ",".join(map(str, exts)) + "):(" + ",".join(map(str, ss)) + ")"
    td = "(" + ",".join(map(str, exts)) + "):(" + ",".join(map(str, sd)) + ")"
    if rng.random() < 0.2 and nd_ >= 64:
        td = "Sw<2,3,3> o " + td
        nd_ = lr.parse(td).cosize  # the library's swizzle-aware bound
    return ts, td, max(ns, O.cosize(O.parse(ts))), nd_


def test_copy_random_pairs(dev, knobs):
    """600 seeded random pairs (permuted, padded, swizzled, 1-16 byte elements, up to
    2^17 elements), each by the default plan, by every path that applies when
    forced, and with 64-bit indices, under randomly drawn plan-time variants
    (access policy, direct loads, tile shape and order, register blocks per lane,
    workgroup lanes, gather grouping, batched swizzles)."""
    rng = random.Random(41)
    runs = 0
    for i in range(600):
        ts, td, ns, nd = _rand_pair(rng)
        eb = rng.choice([1, 2, 4, 8, 16])
        src = np.random.default_rng(i).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        pol = rng.choice([(0, -1), (2, -1), (2, 2), (2, 0)])  # the last: vector/generic paths only
        env = {"load_policy": pol[0], "store_policy": pol[1], "direct_loads": rng.choice([-1, 0, 1]),
               "tile_shape": rng.randint(0, 6) if random.Random(5000 + i).random() > 0.15 else 8,
               "tile_order": rng.randint(0, 9),
               "element_tiles": rng.choice([-1, 0, 1]), "interleave_form": rng.choice([0, 1, 2]),
               "vector_order": rng.choice([-1, 0, 1, 2, 3]), "units_per_lane": rng.choice([-1, 1, 4]),
               "gather_chunks": rng.choice([-1, 1, 2, 4, 8, 16, 32]), "pipeline_tiles": rng.choice([-1, -1, 2, 3, 5]),
               "transpose_reads": rng.choice([-1, 0, 1]),
               "chunk_bytes": random.Random(i).choice([-1, -1, 8, 16]),
               "workgroup_lanes": random.Random(1000 + i).choice([-1, 64, 128, 256]),
               "batch_swizzle": random.Random(2000 + i).choice([-1, -1] + list(range(16))),
               "batch_order": random.Random(3000 + i).choice([-1, 0, 1]),
               "transpose_blocks": random.Random(4000 + i).choice([-1, 1, 2])}
        knobs.t.clear()
        knobs.set(**env)
        if i % 50 == 0:
            say("copy random", i, ts, "->", td, "eb", eb, env)
        for flags in [0, lr.COPY_WIDE_INDEX] + [lr.COPY_FORCE_PATH(p) for p in ALL_PATHS]:
            try:
                p = plan(ts, ns, td, nd, eb, flags)
            except lr.LayoutRemapError as e:
                # a forced path that does not apply, or loads and stores apart on a
                # path other than vector/generic
                assert e.code == lr.binding.ERR_PATH and (flags or pol == (2, 0))
                continue
            got = gpu_copy(dev, src, ts, dst, td, eb, flags)
            assert np.array_equal(got, want), (i, ts, td, eb, hex(flags), env, p["path"])
            runs += 1
    assert runs > 3000


def _write_counts(dev, src, ts, dst, td, eb, flags=0):
    s = torch.from_numpy(src).to(dev)
    d = torch.from_numpy(dst).to(dev)
    counts = torch.zeros(dst.nbytes // eb, dtype=torch.int32, device=dev)
    lr.layout_copy_count_writes(s, ts, d, td, counts, elem_bytes=eb, flags=flags, tuning=KNOBS.tuning())
    torch.cuda.synchronize()
    return d.cpu().numpy(), counts.cpu().numpy()


def _multiplicity(Ld, n, nd):
    """How many logical indices the oracle sends to each destination offset."""
    return np.bincount(O.eval_indices(Ld, np.arange(n)), minlength=nd)


def test_write_counts_random_pairs_and_aliased_tile(dev, knobs):
    """The kernels store every destination element exactly once: each offset the
    oracle's copy writes (multiplicity >= 1) is stored once, every other offset
    never -- on random pairs under the default plan, every forced path and random
    tuning, and on the aliased 8x8 tile, where offsets 16..31 have multiplicity two
    and only the last writer stores.  The copied bytes are checked too."""
    w = W.tile8x8()
    src, dst = W.make_src(w), W.make_dst(w)
    Ld = O.parse(w.dst_layout)
    mult = _multiplicity(Ld, 64, 64)
    assert mult[16:32].tolist() == [2] * 16 and mult[48:].tolist() == [0] * 16
    got, counts = _write_counts(dev, src, w.src_layout, dst, w.dst_layout, 4, lr.COPY_ORDERED_ALIAS)
    assert np.array_equal(counts, (mult > 0).astype(np.int32))
    assert np.array_equal(got, O.copy(src, O.parse(w.src_layout), dst, Ld, 4, ordered_alias=True))
    rng = random.Random(77)
    runs = 0
    for i in range(150):
        ts, td, ns, nd = _rand_pair(rng)
        eb = rng.choice([1, 2, 4, 8, 16])
        src = np.random.default_rng(1000 + i).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        Ls, Ld = O.parse(ts), O.parse(td)
        want = O.copy(src, Ls, dst, Ld, eb)
        mult = _multiplicity(Ld, O.size(Ls), nd)
        knobs.t.clear()
        knobs.set(tile_shape=rng.choice([0, 1, 2, 3, 4, 5, 6, 8]), tile_order=rng.randint(0, 9), gather_chunks=rng.choice([-1, 8, 16]),
                  vector_order=rng.choice([-1, 0, 1, 2, 3]), element_tiles=rng.choice([-1, 0, 1]),
                  pipeline_tiles=rng.choice([-1, 2, 3]), transpose_reads=rng.choice([-1, 1]),
                  direct_loads=rng.choice([-1, 1]), transpose_blocks=random.Random(6000 + i).choice([-1, 2]))
        for flags in [0] + [lr.COPY_FORCE_PATH(p) for p in ALL_PATHS]:
            try:
                p = plan(ts, ns, td, nd, eb, flags)
            except lr.LayoutRemapError as e:
                assert e.code == lr.binding.ERR_PATH and flags
                continue
            got, counts = _write_counts(dev, src, ts, dst, td, eb, flags)
            assert np.array_equal(counts, mult), (i, ts, td, eb, p["path"])
            assert np.array_equal(got, want), (i, ts, td, eb, p["path"])
            runs += 1
        if i % 50 == 0:
            say("write counts", i, ts, "->", td, "eb", eb)
    assert runs > 600


@pytest.mark.slow
@pytest.mark.parametrize("name", ["transpose", "retile", "interleave", "interleave_cm", "nhwc2nchw", "padtiles",
                                  "head_split"])
def test_write_counts_full_size(dev, name):
    """At full size, in the launch configuration the benchmark times: the
    destination layouts are bijections onto [0, N) (the oracle's injectivity test
    and cosize == size), so a correct copy stores every element exactly once."""
    w = W.full(name)
    Ld = O.parse(w.dst_layout)
    assert O.is_injective(Ld) and O.cosize(Ld) == w.n_elems == w.dst_elems
    s = torch.randint(0, 256, (w.src_elems * w.elem_bytes,), dtype=torch.uint8, device=dev)
    d = torch.empty(w.dst_elems * w.elem_bytes, dtype=torch.uint8, device=dev)
    counts = torch.zeros(w.dst_elems, dtype=torch.int32, device=dev)
    say("write counts full", w.name, plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, w.elem_bytes)["path"])
    lr.layout_copy_count_writes(s, w.src_layout, d, w.dst_layout, counts, elem_bytes=w.elem_bytes)
    torch.cuda.synchronize()
    assert int(counts.min()) == 1 and int(counts.max()) == 1
    del s, d, counts
    torch.cuda.empty_cache()


def test_copy_misaligned_pointers(dev):
    w = W.small("retile")
    src, dst, want = _oracle_copy(w)
    for so, do in [(2, 0), (0, 4), (8, 8), (6, 2)]:
        say("copy misaligned", so, do)
        got = gpu_copy(dev, src, w.src_layout, dst, w.dst_layout, 2, 0, src_off=so, dst_off=do)
        assert np.array_equal(got, want)


def test_copy_size_one_and_rank16(dev):
    say("copy size one")
    src = np.arange(16, dtype=np.uint8)
    got = gpu_copy(dev, src, "1:0", np.full(4, 0xA5, np.uint8), "(1,1):(0,0)", 4)
    assert got.tolist() == [0, 1, 2, 3]
    say("copy rank 16")
    ts = "(" + ",".join(["2"] * 16) + "):(" + ",".join(str(1 << i) for i in range(16)) + ")"
    td = "(" + ",".join(["2"] * 16) + "):(" + ",".join(str(1 << (15 - i)) for i in range(16)) + ")"
    src = np.random.default_rng(3).integers(0, 256, (1 << 16) * 2, dtype=np.uint8)
    dst = np.full((1 << 16) * 2, 0xA5, np.uint8)
    want = O.copy(src, O.parse(ts), dst, O.parse(td), 2)
    assert np.array_equal(gpu_copy(dev, src, ts, dst, td, 2), want)


def test_copy_errors(dev):
    say("copy errors")
    t = torch.zeros(256, dtype=torch.uint8, device=dev)
    with pytest.raises(lr.LayoutRemapError) as e:
        lr.layout_copy(t[:128], "32:1", t[64:], "32:1", elem_bytes=4)
    assert e.value.code == lr.binding.ERR_OVERLAP
    with pytest.raises(lr.LayoutRemapError) as e:
        lr.layout_copy(t[:128], "33:1", t[128:], "33:1", elem_bytes=4)
    assert e.value.code == lr.binding.ERR_BOUNDS
    with pytest.raises(lr.LayoutRemapError) as e:
        lr.layout_copy(t[:128], "(4,8):(1,4)", t[128:], "(4,8):(1,0)", elem_bytes=4)
    assert e.value.code == lr.binding.ERR_ALIAS


def test_copy_ordered_alias_larger(dev):
    # several 8192-offset windows, many writers per offset
    say("copy ordered alias")
    ts, td = "(300,50):(1,300)", "(300,50):(7,100)"
    Ls, Ld = O.parse(ts), O.parse(td)
    src = np.random.default_rng(8).integers(0, 256, 15000 * 4, dtype=np.uint8)
    dst = np.full(O.cosize(Ld) * 4, 0xA5, np.uint8)
    want = O.copy(src, Ls, dst, Ld, 4, ordered_alias=True)
    got = gpu_copy(dev, src, ts, dst, td, 4, lr.COPY_ORDERED_ALIAS)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# Full sizes, in the launch configuration bench.py times
# ---------------------------------------------------------------------------
FORMS = {
    "transpose": lambda s: F.transpose(s, 8192),
    "retile": lambda s: F.retile(s, 4096),
    "interleave": lambda s: F.interleave(s, 16, 32, 4096, 128),
    "interleave_cm": lambda s: F.interleave_cm(s, 16, 32, 4096, 128),
    "nhwc2nchw": lambda s: F.nhwc2nchw(s, 128, 56, 56, 256),
    "padtiles": lambda s: F.padtiles(s, 1 << 20),
    "shard_pack": lambda s: F.shard_pack(s, 1024, 8192, 8),
    "rgb_nhwc2nchw": lambda s: F.nhwc2nchw(s, 512, 224, 224, 3),
    "head_split": lambda s: F.head_split(s, 16, 4096, 32, 128),
}

FULL_PATH = {"transpose": "transpose", "retile": "vector", "interleave": "interleave", "interleave_cm": "transpose",
             "nhwc2nchw": "transpose", "padtiles": "staged", "shard_pack": "transpose",
             "rgb_nhwc2nchw": "deinterleave", "head_split": "vector"}


@pytest.mark.slow
@pytest.mark.parametrize("name", list(FORMS))
def test_full_size(dev, name):
    w = W.full(name)
    say("full", w.name, "generate")
    src = W.make_src(w)
    Ls, Ld = O.parse(w.src_layout), O.parse(w.dst_layout)
    p = plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, w.elem_bytes)
    assert p["path"] == FULL_PATH[name]
    s = torch.from_numpy(src).to(dev)
    d = torch.full((w.dst_elems * w.elem_bytes,), 0xA5, dtype=torch.uint8, device=dev)
    say("full", w.name, "copy", p["path"])
    copy_(s, w.src_layout, d, w.dst_layout, w.elem_bytes)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    del s, d
    # sampled indices against the oracle's own evaluation
    ks = np.random.default_rng(7).integers(0, w.n_elems, 1 << 20, dtype=np.int64)
    assert O.copy_sampled_check(src, Ls, got, Ld, w.elem_bytes, ks) == 0
    # the whole buffer against the NumPy closed form
    say("full", w.name, "compare")
    assert np.array_equal(got, FORMS[name](src))


@pytest.mark.slow
@pytest.mark.parametrize("nt", ["0", "1"])
def test_full_transpose_both_variants(dev, knobs, nt):
    # plain and streaming (non-temporal) accesses; the default for this size is streaming
    knobs.policy(nt)
    w = W.full("transpose")
    p = plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    assert p["streaming"] == (nt == "1") and p["store_policy"] == (18 if nt == "1" else 0)
    src = W.make_src(w)
    want = F.transpose(src, 8192)
    s = torch.from_numpy(src).to(dev)
    for path in (lr.PATH_TRANSPOSE, lr.PATH_TRANSPOSE_DIRECT):
        say("full transpose", lr.binding.PATH_NAMES[path], "nt", nt)
        d = torch.full((w.dst_elems * 2,), 0xA5, dtype=torch.uint8, device=dev)
        copy_(s, w.src_layout, d, w.dst_layout, 2, lr.COPY_FORCE_PATH(path))
        torch.cuda.synchronize()
        assert np.array_equal(d.cpu().numpy(), want)


# transposes whose default tiles come from the tile-shape rules for 8- and 16-byte
# elements and for whole blocks: (source, destination, element bytes, tile, closed form)
TILE_RULE_CASES = {
    "fp64 4096x8192": ("(4096,8192):(8192,1)", "(4096,8192):(1,4096)", 8, (32, 64),
                       lambda s: F.transpose_batched(s, 1, 4096, 8192, 8)),
    "16-byte 4096^2": ("(4096,4096):(4096,1)", "(4096,4096):(1,4096)", 16, (64, 16),
                       lambda s: F.transpose_batched(s, 1, 4096, 4096, 16)),
    "NCHW->NHWC (128,256,56,56)": ("(128,3136,256):(802816,1,3136)", "(128,3136,256):(802816,256,1)", 2,
                                   (64, 256), lambda s: F.nchw2nhwc(s, 128, 56, 56, 256, 2)),
    "fp32 128x96 x 4096": ("(128,96,4096):(96,1,12288)", "(128,96,4096):(1,128,12288)", 4, (32, 128),
                           lambda s: F.transpose_batched(s, 4096, 128, 96, 4)),
}


@pytest.mark.slow
@pytest.mark.parametrize("case", list(TILE_RULE_CASES))
def test_full_size_tile_rule_transposes(dev, case):
    """Full-size parity of the transposes whose tiles the planner picks by element size
    (16 x 32 chunks for 8-byte elements, 64 x 16 for 16-byte ones) and by whole blocks
    (8 x 32 chunks where each tile writes one contiguous destination block): the whole
    destination buffer against the oracle's closed forms."""
    ts, td, eb, tile, form = TILE_RULE_CASES[case]
    n = lr.parse(ts).size
    p = plan(ts, n, td, n, eb)
    assert p["path"] == "transpose" and (p["tile_a"], p["tile_b"]) == tile, p
    src = np.random.default_rng(len(case)).integers(0, 256, n * eb, dtype=np.uint8)
    s = torch.from_numpy(src).to(dev)
    d = torch.full((n * eb,), 0xA5, dtype=torch.uint8, device=dev)
    say("full tile-rule transpose", case, "tile", tile)
    copy_(s, ts, d, td, eb)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    del s, d
    torch.cuda.empty_cache()
    assert np.array_equal(got, form(src)), case


def _flat(text):
    """'(a,b,...):(x,y,...)' -> shape and strides (flat layouts without swizzle)."""
    sh, st = text.split(":")
    return [int(v) for v in sh.strip("()").split(",")], [int(v) for v in st.strip("()").split(",")]


@pytest.mark.slow
@pytest.mark.parametrize("k", range(16))
def test_layout_sweep_transforms_full_size(dev, k):
    """Every transform the layout sweep times (bench.py LAYOUT_SWEEP), at its full size in the
    plan the planner picks: the whole destination buffer, holes included, against the
    oracle's strided-copy form (pinned to oracle.copy)."""
    import bench
    name, ts, td, eb = bench.LAYOUT_SWEEP[k]
    Ls, Ld = lr.parse(ts), lr.parse(td)
    n, ns, nd = Ls.size, Ls.cosize, Ld.cosize
    p = plan(ts, ns, td, nd, eb)
    src = np.random.default_rng(900 + k).integers(0, 256, ns * eb, dtype=np.uint8)
    dst = np.full(nd * eb, 0xA5, np.uint8)
    s = torch.from_numpy(src).to(dev)
    d = torch.from_numpy(dst).to(dev)
    say("layout sweep transform", k, name, p["path"], p["tile_a"], p["tile_b"])
    copy_(s, ts, d, td, eb)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    del s, d
    torch.cuda.empty_cache()
    shape, ss = _flat(ts)
    shape_d, sd = _flat(td)
    assert shape == shape_d
    assert np.array_equal(got, F.strided_copy(src, shape, ss, dst, sd, eb)), name


def _rand_flat_large(rng):
    """A random pair of flat layouts over 2^21-2^25 elements: rank 2-4, a random
    mode order on each side, rows padded at random on either side, extents ragged
    against every tile (odd factors)."""
    rank = rng.randint(2, 4)
    total_log = rng.randint(21, 25)
    ext = []
    left = total_log
    for k in range(rank - 1):
        e = rng.randint(3, max(3, left - 2 * (rank - 1 - k)))
        ext.append(e)
        left -= e
    ext.append(max(1, left))
    shape = [(1 << e) + rng.choice([0, 0, 0, -1, 1, 3, -3, 7]) for e in ext]
    shape = [max(2, s) for s in shape]

    def strides(order, pad):
        st = [0] * rank
        acc = 1
        for k in order:
            st[k] = acc
            acc *= shape[k] + (rng.choice([0, 0, 1, 8, 13]) if pad and k == order[0] else 0)
        return st

    src_order = list(range(rank))
    dst_order = list(range(rank))
    rng.shuffle(dst_order)
    if rng.random() < 0.3:
        rng.shuffle(src_order)
    return shape, strides(src_order, True), strides(dst_order, rng.random() < 0.5)


@pytest.mark.slow
def test_random_large_flat_copies(dev, knobs):
    """24 seeded random pairs of flat layouts at 2^21-2^25 elements and 1- to 16-byte
    elements (transposes, permutes, padded rows on either side, ragged extents) under
    the planner's default plan: whole destination buffers, holes included, against
    the oracle's strided-copy form."""
    rng = random.Random(2024)
    for i in range(24):
        shape, ss, sd = _rand_flat_large(rng)
        eb = rng.choice([1, 2, 4, 8, 16])
        while eb > 1 and np.prod(shape) * eb > (1 << 27):
            eb //= 2
        ts = "(" + ",".join(map(str, shape)) + "):(" + ",".join(map(str, ss)) + ")"
        td = "(" + ",".join(map(str, shape)) + "):(" + ",".join(map(str, sd)) + ")"
        ns = 1 + sum((e - 1) * x for e, x in zip(shape, ss))
        nd = 1 + sum((e - 1) * x for e, x in zip(shape, sd))
        p = plan(ts, ns, td, nd, eb)
        say("random large", i, ts, "->", td, "eb", eb, p["path"], p["tile_a"], p["tile_b"])
        src = np.random.default_rng(3000 + i).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        s = torch.from_numpy(src).to(dev)
        d = torch.from_numpy(dst).to(dev)
        copy_(s, ts, d, td, eb)
        torch.cuda.synchronize()
        got = d.cpu().numpy()
        del s, d
        assert np.array_equal(got, F.strided_copy(src, shape, ss, dst, sd, eb)), (i, ts, td, eb)
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_copy_beyond_2_31_elements(dev):
    """More than 2^31 elements: by default the copy is cut into blocks that each fit
    32-bit offsets (launched at offset base pointers); with LR_COPY_WIDE_INDEX it is
    one launch with 64-bit index arithmetic."""
    N = 715827883                      # 3 * N = 2^31 + 1
    M = 46400                          # M^2 > 2^31, blocks of 23232 and 23168 rows
    cases = [(f"(3,{N}):({N},1)", f"(3,{N}):(1,3)", 3 * N, lambda s: s.reshape(3, N).T.reshape(-1), "interleave", 0),
             (f"{(1 << 31) + 16}:1", f"{(1 << 31) + 16}:1", (1 << 31) + 16, lambda s: s, "vector", 0),
             (f"{(1 << 31) + 16}:1", f"{(1 << 31) + 16}:1", (1 << 31) + 16, lambda s: s, "vector",
              lr.COPY_WIDE_INDEX),
             (f"({M},{M}):({M},1)", f"({M},{M}):(1,{M})", M * M, lambda s: s.reshape(M, M).T.reshape(-1),
              "transpose", 0)]
    for ts, td, n, form, path, flags in cases:
        p = plan(ts, n, td, n, 1, flags)
        assert p["path"] == path and (p["wide"] if flags else p["blocks"] > 1), p
        say("beyond 2^31", ts, "->", td, p["path"], "vec", p["vec_elems"], "blocks", p["blocks"], "wide", p["wide"])
        src = np.random.default_rng(n % 1000).integers(0, 256, n, dtype=np.uint8)
        s = torch.from_numpy(src).to(dev)
        d = torch.full((n,), 0xA5, dtype=torch.uint8, device=dev)
        copy_(s, ts, d, td, 1, flags)
        torch.cuda.synchronize()
        got = d.cpu().numpy()
        del s, d
        torch.cuda.empty_cache()
        ks = np.concatenate([np.random.default_rng(3).integers(0, n, 1 << 18, dtype=np.int64),
                             np.arange(n - 4096, n, dtype=np.int64)])
        assert O.copy_sampled_check(src, O.parse(ts), got, O.parse(td), 1, ks) == 0
        assert np.array_equal(got, form(src))
        del src, got


@pytest.mark.slow
def test_channel_shuffle_destination_beyond_4_gib(dev):
    """fp32 RGB images (7200,224,224,3), 4.3 GB each way: element offsets stay under
    2^31 (one launch, 32-bit element arithmetic) while destination byte offsets pass
    4 GiB.  The de-interleave (NHWC -> NCHW) and the channel-shuffle interleave
    (NCHW -> NHWC) must not wrap their stores at 4 GiB: whole buffers against the
    NumPy closed forms.  The source is every element's own index, so a misplaced
    element cannot match."""
    n, h, w, c = 7200, 224, 224, 3
    hw = h * w
    N = n * hw * c
    assert N < (1 << 31) and N * 4 > (1 << 32)
    nhwc = f"({n},{h},{w},{c}):({hw * c},{w * c},{c},1)"
    nchw = f"({n},{h},{w},{c}):({hw * c},{w},1,{hw})"
    src = np.arange(N, dtype=np.uint32).view(np.uint8)
    for ts, td, path, form in ((nhwc, nchw, "deinterleave", F.nhwc2nchw), (nchw, nhwc, "interleave", F.nchw2nhwc)):
        p = plan(ts, N, td, N, 4)
        assert p["path"] == path and not p["wide"] and p["blocks"] == 1, p
        say("beyond 4 GiB", path, "store policy", p["store_policy"])
        s = torch.from_numpy(src).to(dev)
        d = torch.full((N * 4,), 0xA5, dtype=torch.uint8, device=dev)
        copy_(s, ts, d, td, 4)
        torch.cuda.synchronize()
        del s
        got = d.cpu().numpy()
        del d
        torch.cuda.empty_cache()
        say("beyond 4 GiB", path, "compare")
        assert np.array_equal(got, form(src, n, h, w, c, 4)), path
        del got


@pytest.mark.parametrize("blocks", [-1, 2])
@pytest.mark.parametrize("nt", ["0", "1"])
def test_copies_replay_in_a_hip_graph(dev, knobs, nt, blocks):
    """lr_layout_copy allocates nothing and records no memset, so captured copies
    (nine copies on six paths in one graph, with plain or streaming accesses, the latter with the
    sc1 buffer stores, and the transposes with one or two register blocks a lane) replay
    correctly; each replay is checked after eager work has changed the sources."""
    knobs.policy(nt)
    knobs.set(transpose_blocks=blocks)
    cases = []
    for name in ("transpose", "retile", "interleave", "nhwc2nchw", "padtiles", "rgb_nhwc2nchw"):
        w = W.small(name)
        cases.append((w.src_layout, w.dst_layout, w.src_elems, w.dst_elems, w.elem_bytes))
    rgb = W.small("rgb_nhwc2nchw")  # and back: the channel-shuffle interleave
    cases.append((rgb.dst_layout, rgb.src_layout, rgb.dst_elems, rgb.src_elems, rgb.elem_bytes))
    cases.append(("(16,16,300):(16,1,256)", "(16,16,300):(1,16,256)", 76800, 76800, 2))  # batched matrices
    cases.append(("(2,320,256):(81920,1,320)", "(2,320,256):(81920,256,1)", 163840, 163840, 2))  # 8 x 32 tiles
    paths = {plan(ts, ns, td, nd, eb)["path"] for ts, td, ns, nd, eb in cases}
    assert {"transpose", "vector", "interleave", "staged", "deinterleave", "batched"} <= paths, paths
    s_list, d_list, plans = [], [], []
    for ts, td, ns, nd, eb in cases:
        s_list.append(torch.zeros(ns * eb, dtype=torch.uint8, device=dev))
        d_list.append(torch.full((nd * eb,), 0xA5, dtype=torch.uint8, device=dev))
        plans.append((ts, td, ns, nd, eb))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            for (ts, td, ns, nd, eb), s, d in zip(plans, s_list, d_list):
                copy_(s, ts, d, td, eb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        srcs = []
        for i, ((ts, td, ns, nd, eb), s) in enumerate(zip(plans, s_list)):
            host = np.random.default_rng(100 * rep + i).integers(0, 256, ns * eb, dtype=np.uint8)
            s.copy_(torch.from_numpy(host).to(dev))   # eager work between replays
            srcs.append(host)
        torch.cuda.synchronize()
        say("graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for (ts, td, ns, nd, eb), host, d in zip(plans, srcs, d_list):
            want = O.copy(host, O.parse(ts), np.full(nd * eb, 0xA5, np.uint8), O.parse(td), eb)
            got = d.cpu().numpy()
            # positions outside the image of td keep what the previous replay left (0xA5 here)
            assert np.array_equal(got, want), (rep, ts)


# ---------------------------------------------------------------------------
# Tuning variants chosen at plan time (tile shapes, narrow-load interleave)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [0, 1, 2, 3, 4, 5, 6, 7, 8])
def test_transpose_tile_shapes(dev, knobs, shape):
    knobs.set(tile_shape=shape)
    for ts, td, n, eb in [("(520,264):(264,1)", "(520,264):(1,520)", 520 * 264, 2),
                          ("(3,7,9,40):(2520,360,40,1)", "(3,7,9,40):(2520,9,1,63)", 7560, 2),
                          ("(100,72):(72,1)", "(100,72):(1,100)", 7200, 4),
                          ("(64,96,5):(96,1,6144)", "(64,96,5):(1,64,6144)", 30720, 8),
                          ("(1024,512):(512,1)", "(1024,512):(1,1024)", 1024 * 512, 2),
                          ("(512,272):(272,1)", "(512,272):(1,512)", 512 * 272, 1)]:
        src = np.random.default_rng(shape).integers(0, 256, n * eb, dtype=np.uint8)
        dst = np.full(n * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for path in (lr.PATH_TRANSPOSE, lr.PATH_TRANSPOSE_DIRECT):
            flags = lr.COPY_FORCE_PATH(path)
            try:
                plan(ts, n, td, n, eb, flags)
            except lr.LayoutRemapError:
                continue
            say("transpose shape", shape, lr.binding.PATH_NAMES[path], ts, "eb", eb)
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb, flags), want)
        for orient in ("0", "1", "2", "3", "4"):
            knobs.set(tile_order=int(orient))
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want)
        knobs.unset("tile_order")


@pytest.mark.parametrize("nt", ["0", "1"])
def test_transpose_two_blocks_per_lane(dev, knobs, nt):
    """transpose_blocks = 2: each lane of the register-loaded LDS transpose moves two
    V x V blocks, so a tile takes half the lanes.  Every tile shape with an even b
    side, ragged tiles on both sides, 1- to 8-byte elements, a grouped b side and a
    swizzled destination, plain and streaming accesses (the latter with the sc1
    buffer stores), and the 8192^2 fp16 transpose at full size."""
    knobs.policy(nt)
    cases = [("(520,264):(264,1)", "(520,264):(1,520)", 520 * 264, 2),
             ("(3,7,9,40):(2520,360,40,1)", "(3,7,9,40):(2520,9,1,63)", 7560, 2),
             ("(100,72):(72,1)", "(100,72):(1,100)", 7200, 4),
             ("(64,96,5):(96,1,6144)", "(64,96,5):(1,64,6144)", 30720, 8),
             ("(1024,512):(512,1)", "Sw<3,3,3> o (1024,512):(1,1024)", 1024 * 512, 2),
             ("(512,272):(272,1)", "(512,272):(1,512)", 512 * 272, 1)]
    for name in ("transpose", "interleave_cm", "nhwc2nchw"):
        w = W.small(name)
        cases.append((w.src_layout, w.dst_layout, max(w.src_elems, w.dst_elems), w.elem_bytes))
    ran = 0
    for ci, (ts, td, n, eb) in enumerate(cases):
        src = np.random.default_rng(300 + ci).integers(0, 256, n * eb, dtype=np.uint8)
        dst = np.full(n * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for shape in range(9):
            knobs.t.clear()
            knobs.policy(nt)
            knobs.set(tile_shape=shape, transpose_blocks=2)
            p = plan(ts, n, td, n, eb)
            if p["path"] != "transpose":
                continue
            two = p["block"] * 2 * p["vec_elems"] ** 2 == p["tile_a"] * p["tile_b"]
            say("two blocks per lane", ts, "->", td, "eb", eb, "shape", shape, "block", p["block"], "two", two)
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, shape)
            ran += two
    assert ran >= 40
    knobs.t.clear()
    knobs.policy(nt)
    knobs.set(transpose_blocks=2)
    w = W.full("transpose")
    assert plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)["block"] == 512
    s = torch.from_numpy(W.make_src(w)).to(dev)
    d = torch.full((w.dst_elems * 2,), 0xA5, dtype=torch.uint8, device=dev)
    say("two blocks per lane: fp16 8192^2")
    copy_(s, w.src_layout, d, w.dst_layout, 2)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), F.transpose(W.make_src(w), 8192))
    del s, d
    torch.cuda.empty_cache()


def test_streaming_accesses_every_path(dev, knobs):
    """Small copies default to plain accesses; a non-temporal load policy forces the
    non-temporal kernels, which must give the same bytes on every path and workload."""
    knobs.policy("1")
    for name in W.FULL:
        w = W.small(name)
        flags = lr.COPY_ORDERED_ALIAS if w.ordered_alias else 0
        p = plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, w.elem_bytes, flags)
        assert p["streaming"] == (p["path"] not in ("alias", "dual")), p["path"]
        src, dst, want = _oracle_copy(w)
        say("streaming small", w.name)
        assert np.array_equal(gpu_copy(dev, src, w.src_layout, dst, w.dst_layout, w.elem_bytes, flags), want)
    for ci, (ts, td, ns, nd, eb) in enumerate(_case_pairs()):
        src = np.random.default_rng(ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for path in ALL_PATHS:
            flags = lr.COPY_FORCE_PATH(path)
            try:
                plan(ts, ns, td, nd, eb, flags)
            except lr.LayoutRemapError:
                continue
            say("streaming path", lr.binding.PATH_NAMES[path], ts, "->", td, "eb", eb)
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb, flags), want)


@pytest.mark.parametrize("tsc1", ["0", "1"])
def test_transpose_streaming_store_forms(dev, knobs, tsc1):
    """Streaming transposes store either with global non-temporal stores or with
    buffer stores relative to each tile's lowest destination offset (nt and sc1
    bits).  Every tile shape, with ragged edges, a batch mode, a grouped b run and
    destination swizzles (the tile base is rounded down past the swizzled bits)."""
    knobs.policy("1", tsc1)
    cm = W.small("interleave_cm")
    cases = [("(520,264):(264,1)", "(520,264):(1,520)", 2),
             ("(3,7,9,40):(2520,360,40,1)", "(3,7,9,40):(2520,9,1,63)", 2),
             ("(1024,512):(512,1)", "Sw<3,3,3> o (1024,512):(1,1024)", 2),
             ("(600,328):(328,1)", "Sw<2,3,5> o (600,328):(1,600)", 2),
             ("(100,72):(72,1)", "Sw<2,2,4> o (100,72):(1,100)", 4),
             ("(64,96,5):(96,1,6144)", "(64,96,5):(1,64,6144)", 8),
             ("(512,272):(272,1)", "(512,272):(1,512)", 1),
             ("(48,80):(80,1)", "(48,80):(1,48)", 16),
             (cm.src_layout, cm.dst_layout, 2)]
    ran = 0
    for shape in range(9):
        knobs.set(tile_shape=shape)
        for ci, (ts, td, eb) in enumerate(cases):
            n = O.size(O.parse(ts))
            ns, nd = max(n, O.cosize(O.parse(ts))), max(n, lr.parse(td).cosize)
            p = plan(ts, ns, td, nd, eb)
            if p["path"] != "transpose":
                continue
            src = np.random.default_rng(ci + 10 * shape).integers(0, 256, ns * eb, dtype=np.uint8)
            dst = np.full(nd * eb, 0xA5, np.uint8)
            want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
            if tsc1 == "1" and p["vec_elems"] * p["elem_bytes"] == 16:
                assert p["store_policy"] == 18, (ts, td, p)
            if tsc1 == "0":
                assert p["store_policy"] == 2
            say("transpose stores", "sc1" if p["store_policy"] == 18 else "global", "shape", shape, ts, "->", td, "eb", eb)
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, td, shape)
            ran += 1
    assert ran >= 40


@pytest.mark.parametrize("sc1", ["0", "1"])
def test_vector_streaming_store_forms(dev, knobs, sc1):
    """The vector path's streaming stores, global nt or buffer stores with nt and sc1
    from the destination base: contiguous, strided, swizzled and retiled layouts with
    ragged unit counts, both traversal orders."""
    knobs.policy("1", sc1)
    rt = W.small("retile")
    cases = [("100000:1", "100000:1", 100000, 2),
             ("(64,130,3):(1,64,8320)", "(64,130,3):(1,200,26000)", 64 * 130 * 3, 2),
             ("(8,4100):(1,8)", "Sw<2,2,3> o (8,4100):(1,8)", 8 * 4100, 4),
             ("(2,777):(1,2)", "(2,777):(1,1600)", 2 * 777, 8),
             ("(1,999):(1,1)", "(1,999):(1,3)", 999, 16),
             (rt.src_layout, rt.dst_layout, rt.n_elems, 2)]
    ran = 0
    for vorder in ("0", "1", "2", "3"):
        knobs.set(vector_order=int(vorder))
        for ci, (ts, td, n, eb) in enumerate(cases):
            ns, nd = max(n, O.cosize(O.parse(ts))), max(n, lr.parse(td).cosize)
            p = plan(ts, ns, td, nd, eb)
            assert p["path"] in ("vector", "generic") and p["vec_elems"] * p["elem_bytes"] == 16, (ts, td, p)
            assert p["store_policy"] == (18 if sc1 == "1" else 2), (ts, td, p)
            src = np.random.default_rng(ci).integers(0, 256, ns * eb, dtype=np.uint8)
            dst = np.full(nd * eb, 0xA5, np.uint8)
            want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
            say("vector stores", "sc1" if sc1 == "1" else "global", ts, "->", td, "eb", eb, "vorder", vorder)
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, td)
            ran += 1
    assert ran == 4 * len(cases)


def _pow2_align(off):
    return 16 if off % 16 == 0 else off & -off


def test_windowed_kernels_misaligned_pointers(dev):
    """The kernels that split each contiguous range into an aligned 16-byte interior
    and single elements at its ends (the channel shuffle for unaligned planes, and
    1-byte element tiles), on buffers starting at element-aligned offsets that are
    not 16-byte aligned; the 2-byte element tiles beside them."""
    def image(n, h, w, c):
        hw = h * w
        return f"({n},{h},{w},{c}):({hw * c},{w * c},{c},1)", f"({n},{h},{w},{c}):({hw * c},{w},1,{hw})"
    ran = 0
    for eb, c in ((2, 3), (1, 3), (4, 2), (1, 8), (8, 2)):
        nhwc, nchw = image(2, 19, 23, c)
        size = 2 * 19 * 23 * c
        src = np.random.default_rng(eb * 10 + c).integers(0, 256, size * eb, dtype=np.uint8)
        dst = np.full(size * eb, 0xA5, np.uint8)
        for ts, td, path in ((nhwc, nchw, "deinterleave"), (nchw, nhwc, "interleave")):
            want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
            for so, do in ((eb, 0), (0, 3 * eb), (5 * eb, 7 * eb)):
                p = plan(ts, size, td, size, eb, src_align=_pow2_align(so), dst_align=_pow2_align(do))
                assert p["path"] == path and p["vec_elems"] == 1, (ts, td, eb, so, do, p)
                say("windowed channel shuffle", path, "eb", eb, "C", c, "offsets", so, do)
                assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb, src_off=so, dst_off=do), want), (ts, eb, so, do)
                ran += 1
    for eb in (1, 2):
        ts, td, n = "(301,517):(517,1)", "(301,517):(1,301)", 301 * 517
        src = np.random.default_rng(40 + eb).integers(0, 256, n * eb, dtype=np.uint8)
        dst = np.full(n * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for so, do in ((eb, 0), (0, 5 * eb), (3 * eb, 11 * eb)):
            p = plan(ts, n, td, n, eb, src_align=_pow2_align(so), dst_align=_pow2_align(do))
            assert p["path"] == "transpose" and p["tile_a"] == 256 // eb and p["block"] == 512, (eb, so, do, p)
            say("element tiles", "eb", eb, "offsets", so, do)
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb, src_off=so, dst_off=do), want), (eb, so, do)
            ran += 1
    assert ran == 36


def test_odd_size_images_full_size(dev):
    """The element-granular channel shuffle at full size, both directions, in the
    plans the planner picks (ordinary accesses below the streaming threshold,
    streaming above it): whole destination buffers against NumPy's permutation."""
    for n, h, w, c, eb, streaming in ((128, 299, 299, 3, 2, False), (64, 331, 331, 4, 2, False),
                                      (256, 299, 299, 3, 1, False), (300, 299, 299, 3, 2, True)):
        hw = h * w
        nhwc = f"({n},{h},{w},{c}):({hw * c},{w * c},{c},1)"
        nchw = f"({n},{h},{w},{c}):({hw * c},{w},1,{hw})"
        size = n * hw * c
        src = np.random.default_rng(n + c + eb).integers(0, 256, size * eb, dtype=np.uint8)
        planar = np.ascontiguousarray(src.reshape(n, h, w, c, eb).transpose(0, 3, 1, 2, 4)).reshape(-1)
        interleaved = np.ascontiguousarray(src.reshape(n, c, h, w, eb).transpose(0, 2, 3, 1, 4)).reshape(-1)
        s = torch.from_numpy(src).to(dev)
        for ts, td, path, want in ((nhwc, nchw, "deinterleave", planar), (nchw, nhwc, "interleave", interleaved)):
            p = plan(ts, size, td, size, eb)
            assert p["path"] == path and p["vec_elems"] == 1 and p["streaming"] == streaming, (n, h, w, c, eb, p)
            say("odd-size image", path, (n, h, w, c), "eb", eb)
            d = torch.full((size * eb,), 0xA5, dtype=torch.uint8, device=dev)
            copy_(s, ts, d, td, eb)
            torch.cuda.synchronize()
            assert np.array_equal(d.cpu().numpy(), want), (path, n, h, w, c, eb)
            del d
        del s


def test_odd_pitch_transposes_full_size(dev):
    """Element-tile transposes at full size in the launch configurations the planner
    picks for them (windowed tiles, ordinary accesses, each workgroup order rule):
    whole destination buffers against NumPy's transpose."""
    cases = [(8191, 8191, 2, 0),    # just short of a multiple of 8 KiB: a fastest
             (8196, 8196, 2, 4),    # just past one: the diagonal with b fastest
             (16383, 4097, 2, 1),   # one pitch just short: b fastest
             (4097, 8193, 4, 4),    # both pitches just past
             (8191, 8191, 1, 0),    # 1-byte elements, two load batches
             (5793, 5793, 8, 0)]
    for r, c, eb, order in cases:
        n = r * c
        ls, ld = f"({r},{c}):({c},1)", f"({r},{c}):(1,{r})"
        p = plan(ls, n, ld, n, eb)
        assert p["path"] == "transpose" and p["vec_elems"] == 1 and p["tile_a"] == 256 // eb, (r, c, eb, p)
        assert p["order"] == order and not p["streaming"], (r, c, eb, p)
        src = np.random.default_rng(r + c + eb).integers(0, 256, n * eb, dtype=np.uint8)
        want = np.ascontiguousarray(src.reshape(r, c, eb).transpose(1, 0, 2)).reshape(-1)
        say("odd-pitch transpose", r, c, "eb", eb, "order", order)
        s = torch.from_numpy(src).to(dev)
        d = torch.full((n * eb,), 0xA5, dtype=torch.uint8, device=dev)
        copy_(s, ls, d, ld, eb)
        torch.cuda.synchronize()
        assert np.array_equal(d.cpu().numpy(), want), (r, c, eb)
        del s, d


def test_small_batched_and_narrow_transposes(dev, knobs):
    """Transposes whose extents leave a tile mostly idle: batches of small matrices
    of 2-byte elements take the batched path, whole matrices per wavefront, and of
    4-byte elements (a quarter of the tile or less) the staged path, one compact
    matrix a block; a short destination-contiguous extent (NCHW -> NHWC with few
    channels) takes tiles no taller than it.  Ragged batches, both policies, and
    every destination element stored once."""
    cases = [("(32,32,300):(32,1,1024)", "(32,32,300):(1,32,1024)", 2, "batched"),
             ("(16,16,1001):(16,1,256)", "(16,16,1001):(1,16,256)", 2, "batched"),
             ("(16,32,257):(32,1,512)", "(16,32,257):(1,16,512)", 2, "batched"),
             ("(32,32,100):(32,1,1024)", "(32,32,100):(1,32,1024)", 4, "staged"),
             ("(16,16,333):(16,1,256)", "(16,16,333):(1,16,256)", 8, "staged"),
             ("(3,1000,32):(32000,1,1000)", "(3,1000,32):(32000,32,1)", 2, "transpose"),
             ("(2,1000,64):(64000,1,1000)", "(2,1000,64):(64000,64,1)", 2, "transpose"),
             ("(2,1000,128):(128000,1,1000)", "(2,1000,128):(128000,128,1)", 2, "transpose"),
             ("(3,221,32):(7072,1,221)", "(3,221,32):(7072,32,1)", 2, "transpose")]
    ran = 0
    for ci, (ts, td, eb, path) in enumerate(cases):
        n = O.size(O.parse(ts))
        ns, nd = max(n, O.cosize(O.parse(ts))), max(n, O.cosize(O.parse(td)))
        src = np.random.default_rng(500 + ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        mult = _multiplicity(O.parse(td), n, nd)
        for nt in ("0", "1"):
            knobs.t.clear()
            knobs.policy(nt)
            p = plan(ts, ns, td, nd, eb)
            assert p["path"] == path, (ts, p)
            say("small/narrow transpose", ts, "eb", eb, "nt", nt, p["path"], p["tile_a"], p["tile_b"])
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, nt)
            got, counts = _write_counts(dev, src, ts, dst, td, eb)
            assert np.array_equal(counts, (mult > 0).astype(np.int32)), ts
            ran += 1
    assert ran == 2 * len(cases)


def test_transpose_xcd_grouped_orders(dev, knobs):
    """Tile orders 5..9: orders 0..4 over workgroup numbers renumbered by XCD (each XCD
    a contiguous run; grids that are and are not multiples of 8).  Chunk tiles of
    every read-back form, element tiles and the register-only transpose; every
    destination element stored once."""
    cases = _pipe_cases() + [("(301,517):(517,1)", "(301,517):(1,301)", 301 * 517, 301 * 517, 2)]
    ran = 0
    for ci, (ts, td, ns, nd, eb) in enumerate(cases):
        src = np.random.default_rng(400 + ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        mult = _multiplicity(O.parse(td), O.size(O.parse(ts)), nd)
        for order in (5, 6, 7, 8, 9):
            for extra, flags in (({}, 0), ({"direct_loads": 1, "tile_shape": 1}, 0),
                                 ({"direct_loads": 1, "transpose_reads": 1}, 0), ({"element_tiles": 1}, 0),
                                 ({}, lr.COPY_FORCE_PATH(lr.PATH_TRANSPOSE_DIRECT))):
                knobs.t.clear()
                knobs.set(tile_order=order, **extra)
                try:
                    p = plan(ts, ns, td, nd, eb, flags)
                except lr.LayoutRemapError:
                    continue
                if not p["path"].startswith("transpose"):
                    continue
                say("xcd order", order, extra, hex(flags), ts, "eb", eb, "grid", p["grid"], "order", p["order"])
                assert p["order"] in (order, order - 1), p   # 8 falls back to 7 without 4 | tiles
                assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb, flags), want), (ts, order, extra)
                if order == 6 and not flags:
                    _, counts = _write_counts(dev, src, ts, dst, td, eb)
                    assert np.array_equal(counts, (mult > 0).astype(np.int32)), (ts, extra)
                ran += 1
    assert ran >= 150


@pytest.mark.parametrize("eb", [1, 2, 4, 8])
def test_transpose_element_tiles(dev, knobs, eb):
    """Transposes whose rows allow no aligned 16-byte chunks run element-granular
    tiles: odd and ragged extents, a grouped dst-contiguous run, swizzles, a batch
    mode, both access policies and every workgroup order."""
    cases = [("(301,517):(517,1)", "(301,517):(1,301)", 301 * 517),
             ("(1000,1001):(1001,1)", "(1000,1001):(1,1000)", 1000 * 1001),
             ("(257,3,129):(387,129,1)", "(257,3,129):(1,33153,257)", 257 * 3 * 129),
             ("(5,2,77):(77,385,1)", "(5,2,77):(2,1,10)", 5 * 2 * 77),
             ("(255,255):(255,1)", "Sw<1,0,3> o (255,255):(1,255)", 256 * 255),
             ("(130,66,3):(66,1,8580)", "(130,66,3):(1,130,8580)", 130 * 66 * 3)]
    knobs.set(element_tiles=1)
    ran = 0
    for ci, (ts, td, n) in enumerate(cases):
        ns = max(n, O.cosize(O.parse(ts)))
        nd = max(n, lr.parse(td).cosize)
        src = np.random.default_rng(ci + 10 * eb).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for nt in ("0", "1"):
            knobs.policy(nt)
            for orient in ("0", "1", "2", "3", "4"):
                knobs.set(tile_order=int(orient))
                p = plan(ts, ns, td, nd, eb, lr.COPY_FORCE_PATH(lr.PATH_TRANSPOSE))
                if p["tile_a"] != 256 // eb or p["block"] != 512:
                    continue  # aligned chunks exist: the chunk transpose runs instead
                say("transpose elements", ts, "->", td, "eb", eb, "nt", nt, "order", orient)
                got = gpu_copy(dev, src, ts, dst, td, eb, lr.COPY_FORCE_PATH(lr.PATH_TRANSPOSE))
                assert np.array_equal(got, want), (ts, td, eb, nt, orient)
                ran += 1
    assert ran >= 16


@pytest.mark.parametrize("shape", [0, 1, 2, 3])
def test_transpose_direct_loads(dev, knobs, shape):
    """The transpose with its source tile loaded straight into LDS."""
    knobs.set(direct_loads=1)
    knobs.set(tile_shape=shape)
    cases = [("(520,264):(264,1)", "(520,264):(1,520)", 520 * 264, 2),
             ("(3,7,9,40):(2520,360,40,1)", "(3,7,9,40):(2520,9,1,63)", 7560, 2),
             ("(100,72):(72,1)", "(100,72):(1,100)", 7200, 4),
             ("(64,96,5):(96,1,6144)", "(64,96,5):(1,64,6144)", 30720, 8),
             ("(1024,512):(512,1)", "(1024,512):(1,1024)", 1024 * 512, 2),
             ("(48,80):(80,1)", "(48,80):(1,48)", 3840, 16),
             (W.small("interleave_cm").src_layout, W.small("interleave_cm").dst_layout,
              W.small("interleave_cm").src_elems, 2)]
    ran = 0
    for ci, (ts, td, n, eb) in enumerate(cases):
        src = np.random.default_rng(ci).integers(0, 256, n * eb, dtype=np.uint8)
        dst = np.full(n * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for nt in ("0", "1"):
            knobs.policy(nt)
            for orient in ("0", "1", "2", "3", "4"):
                knobs.set(tile_order=int(orient))
                p = plan(ts, n, td, n, eb)
                if p["path"] != "transpose":
                    continue
                say("transpose direct", shape, ts, "eb", eb, "nt", nt, "order", orient, "tile", p["tile_a"], p["tile_b"])
                assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, nt, orient)
                ran += 1
    assert ran >= 16


@pytest.mark.slow
def test_full_transpose_direct_loads(dev, knobs):
    knobs.set(direct_loads=1)
    w = W.full("transpose")
    src = W.make_src(w)
    s = torch.from_numpy(src).to(dev)
    d = torch.full((w.dst_elems * 2,), 0xA5, dtype=torch.uint8, device=dev)
    say("full transpose direct loads")
    copy_(s, w.src_layout, d, w.dst_layout, 2)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), F.transpose(src, 8192))


def _pipe_cases():
    cm = W.small("interleave_cm")
    cases = [("(520,264):(264,1)", "(520,264):(1,520)", 2),
             ("(2,2,128,40):(10240,5120,40,1)", "(2,2,128,40):(10240,5120,1,128)", 2),
             ("(100,72):(72,1)", "(100,72):(1,100)", 4),
             ("(64,96,5):(96,1,6144)", "(64,96,5):(1,64,6144)", 8),
             ("(1024,512):(512,1)", "Sw<3,3,3> o (1024,512):(1,1024)", 2),
             ("(600,328):(328,1)", "Sw<2,3,5> o (600,328):(1,600)", 2),
             ("(48,80):(80,1)", "(48,80):(1,48)", 16),
             ("(512,272):(272,1)", "(512,272):(1,512)", 1),
             ("(3,96,400):(38400,400,1)", "(3,96,400):(38400,1,96)", 1),
             ("(640,320):(320,1)", "Sw<2,4,4> o (640,320):(1,640)", 1),
             (cm.src_layout, cm.dst_layout, 2)]
    out = []
    for ts, td, eb in cases:
        n = O.size(O.parse(ts))
        out.append((ts, td, max(n, O.cosize(O.parse(ts))), max(n, lr.parse(td).cosize), eb))
    return out


@pytest.mark.parametrize("shape", [0, 1, 2])
def test_transpose_pipelined(dev, knobs, shape):
    """The software-pipelined transpose: a workgroup takes pipeline_tiles tiles in
    turn over two LDS tiles.  Tile counts that leave the last workgroup one tile,
    two tiles or a full run; ragged edges, batch modes, a split b mode, 1- to
    16-byte elements; both policies and every tile order."""
    ran = 0
    for ci, (ts, td, ns, nd, eb) in enumerate(_pipe_cases()):
        src = np.random.default_rng(50 + ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for pipe in (2, 3, 4, 7):
            knobs.t.clear()
            knobs.set(tile_shape=shape, pipeline_tiles=pipe)
            for nt in ("0", "1"):
                knobs.policy(nt)
                for orient in ("0", "1", "2", "3", "4"):
                    knobs.set(tile_order=int(orient))
                    p = plan(ts, ns, td, nd, eb)
                    if p["path"] != "transpose" or p["pipeline_tiles"] != pipe:
                        continue
                    assert p["direct"]
                    say("transpose pipelined", shape, pipe, ts, "eb", eb, "nt", nt, "order", orient, "grid", p["grid"])
                    assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, pipe, nt, orient)
                    ran += 1
    assert ran >= 60


@pytest.mark.parametrize("shape", [0, 1, 2, 3])
def test_transpose_reads(dev, knobs, shape):
    """The LDS tile read back with the gfx950 transpose reads (ds_read_b64_tr_b16 and
    ds_read_b64_tr_b8), one tile per workgroup and pipelined: 2- and 1-byte elements,
    ragged edges, batch modes, a grouped b run, destination swizzles; both policies and
    every tile order."""
    ran = {1: 0, 2: 0}
    for ci, (ts, td, ns, nd, eb) in enumerate(_pipe_cases()):
        if eb > 2:
            continue
        src = np.random.default_rng(70 + ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for pipe in (0, 3):
            knobs.t.clear()
            knobs.set(tile_shape=shape, transpose_reads=1, direct_loads=1)
            if pipe:
                knobs.set(pipeline_tiles=pipe)
            for nt in ("0", "1"):
                knobs.policy(nt)
                for orient in ("0", "1", "2", "3", "4"):
                    knobs.set(tile_order=int(orient))
                    p = plan(ts, ns, td, nd, eb)
                    if p["path"] != "transpose" or not p["transpose_reads"]:
                        continue
                    say("transpose reads", shape, pipe, ts, "eb", eb, "nt", nt, "order", orient, "grid", p["grid"])
                    assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, pipe, nt, orient)
                    ran[eb] += 1
    assert ran[2] >= (40 if shape < 3 else 20)
    assert ran[1] >= (20 if shape == 0 else 10)  # 16 x 16-byte chunks: 32 x 32 does not fit, no pipelined 32 x 16


def test_workgroup_lanes(dev, knobs):
    """64-, 128- and 256-lane workgroups on the streaming kernels with one unit per lane:
    vector copies with ragged unit counts and several modes, 2- to 16-byte units, both
    policies, and the narrow interleave at every short extent."""
    cases = [("(1000003):(1)", "(1000003):(1)", 2), ("(8,7,1001):(1,8,56)", "(8,7,1001):(1,8008,8)", 2),
             ("(64,3,333):(1,64,192)", "(64,3,333):(1,21312,64)", 4), ("(5000,3):(1,5000)", "(5000,3):(3,1)", 16),
             ("(128,50,7):(1,128,6400)", "(128,50,7):(1,896,128)", 2)]
    for eb, nb in [(2, 2), (2, 4), (2, 8), (4, 2), (4, 4), (8, 2), (1, 16)]:
        a, bt = 16 // eb * 37 + (16 // eb) * 3, 5
        cases.append((f"({nb},{a},{bt}):({a},1,{a * nb})", f"({nb},{a},{bt}):(1,{nb},{a * nb})", eb))
    # the channel shuffle, both directions: 3 and 4 channels, ragged pixel counts
    for eb, c, px in [(2, 3, 8 * 700), (4, 3, 4 * 333), (1, 4, 16 * 301), (2, 5, 8 * 129)]:
        nhwc, nchw = f"({c},{px},3):(1,{c},{c * px})", f"({c},{px},3):({px},1,{c * px})"
        cases += [(nhwc, nchw, eb), (nchw, nhwc, eb)]
    ran = 0
    for ci, (ts, td, eb) in enumerate(cases):
        ns, nd = lr.parse(ts).cosize, lr.parse(td).cosize
        n = O.size(O.parse(ts))
        ns, nd = max(ns, n), max(nd, n)
        src = np.random.default_rng(210 + ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for lanes in (64, 128, 256):
            for nt in ("0", "1"):
                knobs.t.clear()
                knobs.set(workgroup_lanes=lanes)
                knobs.policy(nt)
                p = plan(ts, ns, td, nd, eb)
                say("workgroup lanes", lanes, ts, "eb", eb, "nt", nt, p["path"], "block", p["block"], "grid", p["grid"])
                assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, lanes, nt)
                if p["block"] == lanes and lanes != 256:
                    ran += 1
    assert ran >= 64  # 64 and 128 lanes, both policies: 2 vector / generic cases, 7 interleaves, 8 shuffles


def test_byte_transpose_chunks(dev, knobs):
    """1-byte transposes in 8- and 16-byte chunks (chunk_bytes), through registers and
    with direct loads, in every tile shape that fits: ragged edges, a batch mode and a
    destination swizzle."""
    ran = 0
    cases = [c for c in _pipe_cases() if c[4] == 1] + [
        ("(1000,528):(528,1)", "(1000,528):(1,1000)", 1000 * 528, 1000 * 528, 1)]
    for ci, (ts, td, ns, nd, eb) in enumerate(cases):
        src = np.random.default_rng(130 + ci).integers(0, 256, ns, dtype=np.uint8)
        dst = np.full(nd, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), 1)
        for cb in (8, 16):
            for shape in range(9):
                for direct in (0, 1):
                    knobs.t.clear()
                    knobs.set(chunk_bytes=cb, tile_shape=shape, direct_loads=direct)
                    p = plan(ts, ns, td, nd, 1)
                    if p["path"] != "transpose":
                        continue
                    assert p["vec_elems"] == cb or cb == 16 and p["vec_elems"] < 16
                    say("byte transpose chunks", ts, "chunk", cb, "shape", shape, "direct", direct, "tile",
                        p["tile_a"], p["tile_b"])
                    assert np.array_equal(gpu_copy(dev, src, ts, dst, td, 1), want), (ts, cb, shape, direct)
                    ran += 1
    assert ran >= 50


def _batched_cases():
    """Batches of small matrices, each compact on both sides: (src, dst, eb)."""
    return [("(16,16,100):(16,1,256)", "(16,16,100):(1,16,256)", 2),
            ("(32,32,9):(32,1,1024)", "(32,32,9):(1,32,1024)", 2),
            ("(64,64,5):(64,1,4096)", "(64,64,5):(1,64,4096)", 2),
            ("(8,8,300):(8,1,64)", "(8,8,300):(1,8,64)", 4),
            ("(16,16,37):(16,1,256)", "(16,16,37):(1,16,256)", 4),
            ("(32,32,7):(32,1,1024)", "(32,32,7):(1,32,1024)", 4),
            ("(24,24,21):(24,1,576)", "(24,24,21):(1,24,576)", 2),
            ("(16,16,19):(16,1,256)", "(16,16,19):(1,16,256)", 8),
            ("(32,32,3):(32,1,1024)", "(32,32,3):(1,32,1024)", 8),
            ("(16,32,13):(32,1,512)", "(16,32,13):(1,16,512)", 2),
            ("(8,16,3,7):(16,1,128,384)", "(8,16,3,7):(1,8,128,384)", 4),
            ("(16,24,7):(24,1,400)", "(16,24,7):(1,16,400)", 2),
            ("(32,16,11):(16,1,520)", "(32,16,11):(1,32,512)", 4),
            ("(136,24):(24,1)", "(136,24):(1,136)", 2)]


def test_batched_small_matrices(dev, knobs):
    """The batched path: whole small matrices per wavefront, square and rectangular,
    counts that leave the last wavefront or workgroup partly empty, padded batch
    strides, two batch modes, one lone matrix; 2-, 4- and 8-byte elements; both
    policies; the planner's own plan too.  Whole buffers against the oracle."""
    force = lr.COPY_FORCE_PATH(lr.PATH_BATCHED)
    for ci, (ts, td, eb) in enumerate(_batched_cases()):
        ns, nd = lr.parse(ts).cosize, lr.parse(td).cosize
        src = np.random.default_rng(150 + ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for nt in ("0", "1"):
            knobs.t.clear()
            knobs.policy(nt)
            p = plan(ts, ns, td, nd, eb, force)
            say("batched", ts, "eb", eb, "nt", nt, "matrices per wave", p["batch_matrices"], "swizzle",
                p["batch_swizzle"], "order", p["batch_order"], "grid", p["grid"])
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb, force), want), (ts, nt)
        knobs.t.clear()
        say("batched, planner's plan", plan(ts, ns, td, nd, eb)["path"])
        assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), ts


@pytest.mark.slow
@pytest.mark.parametrize("count", [4194304, 8388609])
def test_full_batched(dev, count):
    """The batched path at its largest: 2^30 fp16 elements (16 x 16 matrices, 2 GiB each
    way), and 2^31 + 256 elements (4 GiB each way), which the library cuts into two
    launches of 32-bit offsets.  A million sampled outputs against the oracle's own
    evaluation, and the whole destination as a permutation of the source's 2-byte
    values (the histograms of both agree)."""
    ts, td = f"(16,16,{count}):(16,1,256)", f"(16,16,{count}):(1,16,256)"
    n = 256 * count
    p = plan(ts, n, td, n, 2)
    assert p["path"] == "batched" and p["blocks"] == (1 if n < (1 << 31) else 2)
    say("full batched", count, "generate")
    g = torch.Generator(device=dev)
    g.manual_seed(count)
    s = torch.randint(0, 256, (2 * n,), dtype=torch.uint8, device=dev, generator=g)
    d = torch.zeros(2 * n, dtype=torch.uint8, device=dev)
    say("full batched", count, "copy")
    copy_(s, ts, d, td, 2)
    torch.cuda.synchronize()
    src = s.cpu().numpy()
    got = d.cpu().numpy()
    del s, d
    torch.cuda.empty_cache()
    say("full batched", count, "compare")
    ks = np.random.default_rng(11).integers(0, n, 1 << 20, dtype=np.int64)
    assert O.copy_sampled_check(src, O.parse(ts), got, O.parse(td), 2, ks) == 0
    hs = np.bincount(src.view(np.uint16), minlength=1 << 16)
    hg = np.bincount(got.view(np.uint16), minlength=1 << 16)
    assert np.array_equal(hs, hg)


def test_batched_write_counts(dev):
    """Every destination element of a batched copy is stored exactly once."""
    for ci, (ts, td, eb) in enumerate(_batched_cases()):
        ns, nd = lr.parse(ts).cosize, lr.parse(td).cosize
        src = np.random.default_rng(170 + ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        mult = _multiplicity(O.parse(td), O.size(O.parse(ts)), nd)
        say("batched write counts", ts, "eb", eb)
        got, counts = _write_counts(dev, src, ts, dst, td, eb, lr.COPY_FORCE_PATH(lr.PATH_BATCHED))
        assert np.array_equal(counts, (mult > 0).astype(np.int32)), ts
        assert np.array_equal(got, O.copy(src, O.parse(ts), dst, O.parse(td), eb))


def test_transpose_pipelined_write_counts(dev, knobs):
    """Every destination element of a pipelined transpose is stored exactly once."""
    ran = 0
    for ci, (ts, td, ns, nd, eb) in enumerate(_pipe_cases()):
        src = np.random.default_rng(90 + ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        mult = _multiplicity(O.parse(td), O.size(O.parse(ts)), nd)
        for shape, pipe, tr in ((0, 3, 0), (1, 2, 0), (2, 5, 0), (1, 2, 1), (3, 0, 1)):
            knobs.t.clear()
            knobs.set(tile_shape=shape, transpose_reads=tr, direct_loads=1)
            if pipe:
                knobs.set(pipeline_tiles=pipe)
            p = plan(ts, ns, td, nd, eb)
            if p["path"] != "transpose" or p["pipeline_tiles"] != pipe or p["transpose_reads"] != bool(tr):
                continue
            say("pipelined write counts", ts, "eb", eb, "shape", shape, "pipe", pipe, "transpose reads", tr)
            got, counts = _write_counts(dev, src, ts, dst, td, eb)
            assert np.array_equal(counts, (mult > 0).astype(np.int32)), (ts, shape, pipe, tr)
            assert np.array_equal(got, O.copy(src, O.parse(ts), dst, O.parse(td), eb))
            ran += 1
    assert ran >= 20


@pytest.mark.slow
@pytest.mark.parametrize("shape,pipe,tr", [(1, 4, 0), (0, 8, 0), (3, 0, 1), (1, 4, 1)])
def test_full_transpose_pipelined(dev, knobs, shape, pipe, tr):
    knobs.set(tile_shape=shape, transpose_reads=tr, direct_loads=1)
    if pipe:
        knobs.set(pipeline_tiles=pipe)
    w = W.full("transpose")
    p = plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2)
    assert p["pipeline_tiles"] == pipe and p["transpose_reads"] == bool(tr)
    src = W.make_src(w)
    s = torch.from_numpy(src).to(dev)
    d = torch.full((w.dst_elems * 2,), 0xA5, dtype=torch.uint8, device=dev)
    say("full transpose pipelined", shape, pipe, "transpose reads", tr)
    copy_(s, w.src_layout, d, w.dst_layout, 2)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), F.transpose(src, 8192))


@pytest.mark.parametrize("lanes", [64, 128, 256])
@pytest.mark.parametrize("direct", [0, 1])
def test_staged_direct_loads(dev, knobs, direct, lanes):
    """The staged path with its footprint loaded straight into LDS (gfx950 direct
    loads) or through registers; both streaming policies; 64-, 128- and 256-lane
    workgroups (raised to one lane per destination chunk of a tile), under every
    gather grouping the plan admits."""
    knobs.set(direct_loads=direct, workgroup_lanes=lanes)
    cases = [(W.small("padtiles").src_layout, W.small("padtiles").dst_layout, W.small("padtiles").src_elems,
              W.small("padtiles").dst_elems, 4)]
    cases += [c for c in _case_pairs()]
    # padded rows of 2 and 4 KiB: 128 and 256 destination chunks a tile
    cases += [("(512,30):(1,520)", "(512,30):(1,512)", 520 * 30, 512 * 30, 4),
              ("(512,9):(1,516)", "(512,9):(1,512)", 516 * 9, 512 * 9, 8)]
    ran = 0
    for nt in ("0", "1"):
        knobs.policy(nt)
        for ci, (ts, td, ns, nd, eb) in enumerate(cases):
            flags = lr.COPY_FORCE_PATH(lr.PATH_STAGED)
            try:
                plan(ts, ns, td, nd, eb, flags)
            except lr.LayoutRemapError:
                continue
            src = np.random.default_rng(ci).integers(0, 256, ns * eb, dtype=np.uint8)
            dst = np.full(nd * eb, 0xA5, np.uint8)
            want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
            seen = set()
            for gc in (-1, 1, 2, 4, 8, 16, 32):  # every gather grouping the plan admits
                knobs.set(gather_chunks=gc)
                p = plan(ts, ns, td, nd, eb, flags)
                g = p["gather_chunks"]
                if g in seen:
                    continue
                seen.add(g)
                assert p["block"] >= lanes
                say("staged direct", direct, "nt", nt, ts, "->", td, "eb", eb, "gather chunks", g,
                    "block", p["block"], "grid", p["grid"])
                assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb, flags), want), (ts, td, g)
                ran += 1
            knobs.unset("gather_chunks")
    assert ran >= 8


@pytest.mark.parametrize("narrow", [0, 1])
def test_interleave_variants(dev, knobs, narrow):
    """Both load variants at every NB, with plain accesses and with streaming ones
    (the narrow variant's streaming stores as global nt stores or as buffer stores
    with nt and sc1), including a swizzled destination."""
    knobs.set(interleave_form=narrow)
    cases = []
    for eb, nb in [(1, 2), (1, 4), (1, 8), (1, 16), (2, 2), (2, 4), (2, 8), (4, 2), (4, 4), (8, 2)]:
        a, bt = 16 // eb * 40, 3
        cases.append((f"({nb},{a},{bt}):({a},1,{a * nb})", f"({nb},{a},{bt}):(1,{nb},{a * nb})", a * nb * bt, eb))
    cases.append(("(2,6400,3):(6400,1,12800)", "Sw<2,4,3> o (2,6400,3):(1,2,12800)", 2 * 6400 * 3, 2))
    for ci, (ts, td, n, eb) in enumerate(cases):
        nd = max(n, lr.parse(td).cosize)
        src = np.random.default_rng(ci).integers(0, 256, n * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for nt, sc1 in (("0", "1"), ("1", "0"), ("1", "1")):
            knobs.policy(nt, sc1)
            p = plan(ts, n, td, nd, eb)
            assert p["path"] == "interleave"
            assert p["store_policy"] == (0 if nt == "0" else 18 if (sc1 == "1" and narrow) else 2), p
            say("interleave narrow", narrow, ts, "->", td, "eb", eb, "nt", nt, "sc1", sc1)
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, td, nt, sc1)


@pytest.mark.parametrize("pol", [(2, 0), (0, 2), (0, 18)])
def test_vector_split_load_store_policies(dev, knobs, pol):
    """The generic and vector paths with loads and stores under different cache
    policies (non-temporal loads with plain stores, and the reverse), every
    traversal order, 16-byte units and narrower ones."""
    rt = W.small("retile")
    cases = [(rt.src_layout, rt.dst_layout, rt.n_elems, rt.n_elems, 2),
             ("(64,130,3):(1,64,8320)", "(64,130,3):(1,200,26000)", 64 * 130 * 3, 200 * 130 * 3, 2),
             ("(100,7):(3,1000)", "(100,7):(1,100)", 3 * 99 + 6001, 700, 4),
             ("100000:1", "100000:1", 100000, 100000, 1)]
    for ci, (ts, td, ns, nd, eb) in enumerate(cases):
        src = np.random.default_rng(ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for vo in (0, 1, 2, 3):
            knobs.t.clear()
            knobs.set(load_policy=pol[0], store_policy=pol[1], vector_order=vo)
            p = plan(ts, ns, td, nd, eb)
            assert p["path"] in ("vector", "generic") and p["load_policy"] == pol[0], (ts, p)
            say("vector policies", pol, "order", vo, ts, "->", td, "eb", eb, p["path"])
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, td, pol, vo)


def _image(n, h, w, c):
    hw = h * w
    return f"({n},{h},{w},{c}):({hw * c},{w * c},{c},1)", f"({n},{h},{w},{c}):({hw * c},{w},1,{hw})"


@pytest.mark.parametrize("eb", [1, 2, 4, 8])
def test_channel_shuffle(dev, knobs, eb):
    """Few-channel image layouts, NHWC <-> NCHW for every channel count the shuffle
    kernels take (2..8 channels of at most 16 bytes), both access policies: a batch
    mode, workgroups cut short at the end of each image, and the register interleave
    replaced by the shuffle for power-of-two channel counts (interleave_form 2)."""
    ran = 0
    for c in range(2, 9):
        if c * eb > 16:
            continue
        v = 16 // eb
        # 3 images of 80 x (4 v) pixels, 320 blocks of v: two workgroups per image,
        # the second holding 64 of its 256 blocks
        n, h, w = 3, 80, 4 * v
        nhwc, nchw = _image(n, h, w, c)
        size = n * h * w * c
        src = np.random.default_rng(c * 10 + eb).integers(0, 256, size * eb, dtype=np.uint8)
        dst = np.full(size * eb, 0xA5, np.uint8)
        for ts, td, path in ((nhwc, nchw, "deinterleave"), (nchw, nhwc, "interleave")):
            want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
            for nt in ("0", "1"):
                for variant in ("default", "2"):
                    knobs.policy(nt)
                    if variant == "2":
                        knobs.set(interleave_form=2)
                    else:
                        knobs.unset("interleave_form")
                    p = plan(ts, size, td, size, eb)
                    assert p["path"] == path, (ts, td, eb, p["path"])
                    shuffled = path == "deinterleave" or c & (c - 1) or variant == "2"
                    if path == "interleave":
                        assert (p["tile_a"] == 256 * v) == bool(shuffled), p
                    say("channel shuffle", path, "eb", eb, "C", c, "nt", nt, "variant", variant)
                    assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, td, eb, nt, variant)
                    ran += 1
    knobs.unset("interleave_form")
    assert ran >= 8


@pytest.mark.parametrize("eb", [1, 2, 4, 8])
def test_channel_shuffle_any_pixel_count(dev, knobs, eb):
    """The element-granular channel shuffle: images whose pixel count leaves the
    planes without whole 16-byte chunks (odd sizes), every channel count, both
    directions and access policies, with a batch and workgroups cut short."""
    ran = 0
    for c in range(2, 9):
        if c * eb > 16:
            continue
        for n, h, w in ((3, 17, 19), (2, 41, 61)):
            nhwc, nchw = _image(n, h, w, c)
            size = n * h * w * c
            src = np.random.default_rng(c * 100 + eb * 7 + h).integers(0, 256, size * eb, dtype=np.uint8)
            dst = np.full(size * eb, 0xA5, np.uint8)
            for ts, td, path in ((nhwc, nchw, "deinterleave"), (nchw, nhwc, "interleave")):
                want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
                for nt in ("0", "1"):
                    knobs.policy(nt)
                    p = plan(ts, size, td, size, eb)
                    assert p["path"] == path and p["vec_elems"] == 1, (ts, td, eb, p)
                    say("channel shuffle elements", path, "eb", eb, "C", c, (n, h, w), "nt", nt)
                    assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, td, eb, nt)
                    ran += 1
    assert ran >= 8


def _atom_cases():
    """(src, dst, src elems, dst elems, eb): the atom (mode 0) of w elements continued by a
    in the source and by b in the destination -- atoms of 2 to 20 chunks (32-320 bytes,
    powers of two and not), extents that leave ragged tiles and partial rounds of
    lanes, batch modes with padding, swizzles on either side, and the 512^2 retile."""
    rt = W.small("retile")
    cases = [
        ("(64,13,21,3):(1,64,832,20000)", "(64,13,21,3):(1,1344,64,17600)", 2),   # K 8, ragged, batch
        ("(64,40,70):(1,64,2560)", "(64,40,70):(1,4480,64)", 1),                    # K 4, T 16
        ("(16,33,17):(1,16,528)", "(16,33,17):(1,272,16)", 4),                      # K 4, T 16
        ("(32,9,6,2):(1,32,300,2000)", "(32,9,6,2):(1,192,32,1728)", 8),            # K 16, T 4
        ("(20,5,7):(1,20,100)", "(20,5,7):(1,140,20)", 16),                         # K 20, T 4, partial round
        ("(64,16,24):(1,64,1024)", "Sw<2,3,4> o (64,16,24):(1,1536,64)", 2),        # dst swizzle
        ("Sw<1,4,3> o (64,16,24):(1,64,1024)", "(64,16,24):(1,1536,64)", 2),        # src swizzle
        ("(8,17,40,8):(1,8,136,5600)", "(8,17,40,8):(1,320,8,5500)", 8),            # K 4, batch
        ("(16,33,35):(1,16,528)", "(16,33,35):(1,560,16)", 2),                      # K 2 (32-byte atoms)
        ("(24,37,19):(1,24,888)", "(24,37,19):(1,456,24)", 2),                      # K 3 (48 bytes)
        ("(40,13,21,2):(1,40,520,11000)", "(40,13,21,2):(1,840,40,11000)", 2),      # K 5, T 8, batch
        ("(24,19,23):(1,24,456)", "(24,19,23):(1,552,24)", 4),                      # K 6
        ("(56,9,11,3):(1,56,504,5600)", "(56,9,11,3):(1,616,56,5600)", 2),          # K 7, ragged
        ("(20,11,9):(1,20,220)", "(20,11,9):(1,180,20)", 8),                        # K 10
        ("(96,10,9):(1,96,960)", "Sw<1,3,4> o (96,10,9):(1,864,96)", 2),            # K 12, dst swizzle
        (rt.src_layout, rt.dst_layout, 2),
    ]
    out = []
    for ts, td, eb in cases:
        n = O.size(O.parse(ts))
        out.append((ts, td, max(n, O.cosize(O.parse(ts))), max(n, lr.parse(td).cosize), eb))
    return out


def test_atom_tiles(dev, knobs):
    """The vector path's tiles of atoms through LDS (vector order 3, the planner's
    choice for these layouts), under both streaming policies and both store forms,
    byte-exact against the oracle."""
    ran = 0
    for ci, (ts, td, ns, nd, eb) in enumerate(_atom_cases()):
        src = np.random.default_rng(200 + ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        for pol in (None, ("0",), ("1", "1"), ("1", "0")):
            knobs.t.clear()
            if pol:
                knobs.policy(*pol)
            p = plan(ts, ns, td, nd, eb)
            assert p["path"] in ("vector", "generic") and p["vector_order"] == 3, (ts, td, p)
            say("atom tiles", ts, "->", td, "eb", eb, "policy", pol, "tile", p["tile_a"], "grid", p["grid"])
            assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want), (ts, td, pol)
            ran += 1
    assert ran == 4 * len(_atom_cases())


def test_atom_tiles_write_counts(dev, knobs):
    """Every destination element of a tiles-of-atoms copy is stored exactly once."""
    for ci, (ts, td, ns, nd, eb) in enumerate(_atom_cases()):
        src = np.random.default_rng(300 + ci).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        mult = _multiplicity(O.parse(td), O.size(O.parse(ts)), nd)
        assert plan(ts, ns, td, nd, eb)["vector_order"] == 3
        say("atom tiles write counts", ts, "eb", eb)
        got, counts = _write_counts(dev, src, ts, dst, td, eb)
        assert np.array_equal(counts, (mult > 0).astype(np.int32)), ts
        assert np.array_equal(got, O.copy(src, O.parse(ts), dst, O.parse(td), eb))


@pytest.mark.parametrize("vorder", [0, 1, 2, 3])
def test_vector_traversal_orders(dev, knobs, vorder):
    knobs.set(vector_order=vorder)
    cases = [(W.small("retile").src_layout, W.small("retile").dst_layout, 512 * 512, 512 * 512, 2),
             ("(64,64):(64,1)", "Sw<3,3,3> o (64,64):(64,1)", 4096, 4096, 2),
             ("(96,5,3):(1,96,480)", "(96,5,3):(1,288,96)", 1440, 1440, 2),
             ("8192:1", "8192:1", 8192, 8192, 4),
             ("(8,2048):(1,8)", "(8,2048):(1,8)", 16384, 16384, 1),
             ("(16,3,256):(1,4096,16)", "(16,3,256):(1,16,48)", 12288, 12288, 2),
             ("(4,64,7):(1,4,256)", "(4,64,7):(1,28,4)", 1792, 1792, 4)]
    for ts, td, ns, nd, eb in cases:
        src = np.random.default_rng(ns).integers(0, 256, ns * eb, dtype=np.uint8)
        dst = np.full(nd * eb, 0xA5, np.uint8)
        want = O.copy(src, O.parse(ts), dst, O.parse(td), eb)
        say("vector order", vorder, ts, "->", td, "eb", eb, plan(ts, ns, td, nd, eb)["path"])
        assert np.array_equal(gpu_copy(dev, src, ts, dst, td, eb), want)
