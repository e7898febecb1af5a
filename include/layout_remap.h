/*
 * layout_remap.h -- C ABI of the MI355X (gfx950) layout-evaluation and
 * layout-remapping-copy library (liblayout_remap.so).
 *
 * The operations are those of hierarchical "shape:stride" layouts as three web
 * pages describe them; citations name the page and its section:
 *   [ThreadMap page]     CUTLASS 2.x PitchLinearStripminedThreadMap article,
 *                        hotelren.com/news/5252042
 *   [CuTe algebra page]  "CUTE布局代数：GPU张量计算的内存优化革命", jsqmd.com/news/768714
 *   [print_layout page]  "CUTLASS Layout可视化：从print_layout理解GPU内存映射与性能优化",
 *                        codechina.net/article/weixin_30702441/411096
 *
 * Conventions for every entry point:
 *   - Return 0 on success or a negative lr_status.  No C++ exception crosses.
 *   - Descriptors (lr_layout) are plain structs owned by the caller; results are
 *     written to caller-provided structs.  The library never allocates device
 *     memory and keeps no global mutable state (the last HIP error text is kept
 *     per calling thread).
 *   - Device pointers are HIP device memory owned by the caller.  Launches are
 *     asynchronous on the caller's stream (a hipStream_t passed as void*; NULL is
 *     the null stream).  Errors found on the host are returned before any launch.
 *   - Element data are moved as opaque bytes: NaN payloads and any bit pattern
 *     survive unchanged.
 *   - Offsets, strides and capacities are in elements, not bytes.
 */
#ifndef LAYOUT_REMAP_H
#define LAYOUT_REMAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Only the lr_* entry points are exported from the shared library (it is built
 * with -fvisibility=hidden). */
#if defined(__GNUC__)
#pragma GCC visibility push(default)
#endif

#define LR_MAX_LEAVES 16

/* Status codes (negative). */
typedef enum {
  LR_OK = 0,
  LR_ERR_INVALID = -1,           /* bad argument: NULL, rank, extent < 1, negative stride, bad text */
  LR_ERR_SIZE_MISMATCH = -2,     /* size(src layout) != size(dst layout) */
  LR_ERR_BOUNDS = -3,            /* a layout reaches beyond its buffer capacity */
  LR_ERR_OVERFLOW = -4,          /* a size or offset does not fit in int64 */
  LR_ERR_ALIAS = -5,             /* dst layout not injective and LR_COPY_ORDERED_ALIAS not set,
                                    or the ordered aliased copy is beyond its limits */
  LR_ERR_NOT_REPRESENTABLE = -6, /* result of an algebra operation is not a layout */
  LR_ERR_SWIZZLE = -7,           /* swizzle parameters invalid (need B >= 0, M >= 0, S >= B, B+M+S <= 62) */
  LR_ERR_ELEM_BYTES = -8,        /* elem_bytes not one of 1, 2, 4, 8, 16 */
  LR_ERR_HIP = -9,               /* a HIP call failed; lr_last_hip_error() gives its text */
  LR_ERR_PATH = -10,             /* a forced copy path does not apply to these layouts */
  LR_ERR_OVERLAP = -11,          /* source and destination storage overlap */
  LR_ERR_CAPACITY = -12          /* text buffer too small (lr_layout_format) */
} lr_status;

/*
 * Layout descriptor.  [CuTe algebra page, section 2.1] and [print_layout page,
 * sections 2.1 and 3.2]: a layout is a function from logical coordinates to
 * offsets given by a (possibly nested) shape and a congruent stride.  The
 * descriptor keeps the leaves of the nested shape in depth-first order and the
 * bounds of the top-level modes; nesting below the top level only groups leaves
 * and does not change the function, so it is flattened.
 *
 * A 1-D index k is split colexicographically over the leaves (leaf 0 fastest):
 * c_i = (k / prod_{j<i} shape_j) % shape_i, and offset = sum_i c_i * stride_i.
 * [ThreadMap page, sections 1.2 and 2.2] split a thread id the same way, the
 * contiguous part first.
 *
 * Optional Swizzle<B,M,S> [print_layout page, section 4.3] is applied to the
 * final offset o:  o ^ ((o >> S) & (((1 << B) - 1) << M)).  swz_b == 0 means no
 * swizzle.  With S >= B it is a bijection and its own inverse.
 */
typedef struct {
  int32_t nleaves;                 /* 1 .. LR_MAX_LEAVES */
  int32_t nmodes;                  /* 1 .. nleaves: top-level modes */
  int64_t shape[LR_MAX_LEAVES];    /* each >= 1 */
  int64_t stride[LR_MAX_LEAVES];   /* each >= 0 */
  int32_t mode_end[LR_MAX_LEAVES]; /* leaf index one past the end of each top-level mode;
                                      strictly increasing, mode_end[nmodes-1] == nleaves */
  int32_t swz_b, swz_m, swz_s;     /* Swizzle<B,M,S> on the final offset; swz_b == 0: none */
} lr_layout;

/* ---------------------------------------------------------------- text form */

/* Parse "(4,2):(_2,_1)", "((4,2),(2,4)):((2,16),(1,8))", "8:1" or
 * "Sw<3,3,3> o ((128,32),(64,64)):((64,524288),(1,8192))" ([print_layout page,
 * section 3.2] for the printed form; "_" marks a compile-time constant there and
 * is accepted and ignored).  Returns LR_ERR_INVALID on malformed text,
 * LR_ERR_SWIZZLE on bad swizzle parameters. */
int lr_layout_parse(const char* text, lr_layout* out);

/* Write the text form of L into buf (NUL-terminated).  LR_ERR_CAPACITY if cap is
 * too small. */
int lr_layout_format(const lr_layout* L, char* buf, size_t cap);

/* Check a descriptor: ranks, extents >= 1, strides >= 0, mode bounds, swizzle,
 * and that size and the largest linear offset fit in int64 (LR_ERR_OVERFLOW). */
int lr_layout_validate(const lr_layout* L);

/* --------------------------------------------------------------- properties */

/* Number of logical elements: product of the extents. */
int lr_size(const lr_layout* L, int64_t* n);

/* Buffer length the layout needs.  Unswizzled: exact, 1 + sum (shape_i-1)*stride_i.
 * Swizzled: an upper bound, 1 + (m | (2^(M+B) - 1)) where m is the unswizzled
 * largest offset (the swizzle only rewrites bits below M+B). */
int lr_cosize(const lr_layout* L, int64_t* n);

/* --------------------------------------------------------------- algebra */

/* Coalesce: the same function of the 1-D index on [0, size) with extent-1 leaves
 * dropped and neighbours merged when stride[i+1] == shape[i]*stride[i]; each
 * remaining leaf becomes a top-level mode.  The swizzle is kept. */
int lr_coalesce(const lr_layout* in, lr_layout* out);

/* Composition R = A o B, R(c) = A(B(c)) with B's integer offset used as a 1-D
 * index into A ([CuTe algebra page, section 2.2]; a padded A is skipped over as
 * that section describes).  A is coalesced and its last leaf extended without
 * bound.  Each leaf (n:s) of B becomes the leaves of A met by skipping s then
 * taking n, which needs divisibility at every leaf boundary; when A has more
 * than one leaf, B's leaves with n > 1 and s > 0, sorted by stride, must cover
 * disjoint ranges (s_j*n_j <= s_{j+1}) so that no carry crosses between them.
 * The result has B's top-level modes and A's swizzle.  A swizzled B is accepted
 * only when A is the identity n:1.  Otherwise LR_ERR_NOT_REPRESENTABLE. */
int lr_composition(const lr_layout* a, const lr_layout* b, lr_layout* out);

/* Right inverse L' with L(L'(i)) == i for i < size(L') ([CuTe algebra page,
 * section 2.3]: which logical index sits at a given offset).  Built greedily:
 * starting from stride 1, take the leaf whose stride equals the product so far
 * and append (its extent : its colex weight in L).  Extent-1 and stride-0 leaves
 * are ignored.  A swizzled L gives LR_ERR_NOT_REPRESENTABLE (its inverse applies
 * the swizzle first, which a descriptor cannot express). */
int lr_right_inverse(const lr_layout* in, lr_layout* out);

/* zipped_divide by a tiler ([CuTe algebra page, section 3.2]): each top-level
 * mode m of extent n_m splits into a tile part (first tiler[m] elements, in colex
 * order) and a rest part (n_m/tiler[m] tiles); the result has two top-level
 * modes, all tile parts then all rest parts.  ntiler <= nmodes; modes past the
 * tiler are not split (they go whole into the rest part).  tiler[m] must divide
 * n_m, else LR_ERR_NOT_REPRESENTABLE. */
int lr_zipped_divide(const lr_layout* in, const int64_t* tiler, int32_t ntiler, lr_layout* out);

/* Slice ([CuTe algebra page, section 3.2]: one tile of a zipped_divide is the
 * layout with the rest mode fixed at the tile's coordinate and the tile mode left
 * free): fix some coordinates of L, keep the others.  coord has ncoord entries:
 * ncoord == nmodes gives one integer per top-level mode (-1 keeps the whole mode,
 * otherwise a 1-D index within the mode, split colexicographically over its
 * leaves); ncoord == nleaves gives one per leaf (-1 keeps the leaf, otherwise its
 * coordinate).  *out receives the kept leaves, in order, grouped by the top-level
 * mode they came from -- when only one such group is left, each of its leaves is a
 * top-level mode of its own (the tile of a zipped_divide keeps its 2-D shape); 1:0
 * when nothing is kept -- and *offset the offset the fixed
 * coordinates contribute, so that L(c) = *offset + out(c') for every c whose fixed
 * entries equal coord (c' its kept part).  A swizzled L keeps its swizzle when
 * *offset is a multiple of 2^(M+S+B) (the swizzle then acts on the kept part
 * alone); otherwise LR_ERR_NOT_REPRESENTABLE.  A coordinate out of range gives
 * LR_ERR_INVALID. */
int lr_slice(const lr_layout* L, const int64_t* coord, int32_t ncoord, lr_layout* out, int64_t* offset);

/* Complement of A up to size M ([CuTe algebra page, section 3.2]: what a tile
 * leaves over): with A's leaves of extent > 1 and stride > 0 sorted by stride,
 * each stride must be a multiple of the previous leaf's extent * stride
 * (LR_ERR_NOT_REPRESENTABLE otherwise); the result is (d_0 : 1),
 * (d_{i+1}/(n_i d_i) : n_i d_i)..., (ceil(M/(n_k d_k)) : n_k d_k), coalesced, one
 * leaf per top-level mode.  (A, complement(A, M)) is then a bijection onto a
 * prefix [0, M') with M' >= M.  A swizzled A gives LR_ERR_NOT_REPRESENTABLE; M >= 1. */
int lr_complement(const lr_layout* A, int64_t M, lr_layout* out);

/* logical_divide(A, B) = A o (B, complement(B, size(A))): top-level mode 0 is the
 * tile B selects from A, mode 1 enumerates the tiles (CuTe algebra page, section
 * 3.2).  B must be unswizzled; composition rules as lr_composition. */
int lr_logical_divide(const lr_layout* A, const lr_layout* B, lr_layout* out);

/* logical_product(A, B) = (A, complement(A, size(A)*cosize(B)) o B): mode 0 is A,
 * mode 1 places one copy of A at each position B describes.  Unswizzled A and B. */
int lr_logical_product(const lr_layout* A, const lr_layout* B, lr_layout* out);

/* blocked_product(A, B): the logical product regrouped mode by mode, top-level
 * mode i = (A's mode i, the copies' mode i) -- [CuTe algebra page, section 4.1]: a
 * 4x8 block over a 2x5 grid gives a "4x2, 8x5" layout.  A and B need the same
 * number of top-level modes (LR_ERR_INVALID otherwise). */
int lr_blocked_product(const lr_layout* A, const lr_layout* B, lr_layout* out);

/* Injectivity of L as a function of the 1-D index.  With the leaves of extent > 1
 * sorted by stride, a leaf whose stride exceeds the largest offset of the smaller
 * ones is separated (its copies of their image cannot meet), so L is injective
 * exactly when the leaves up to the last one that is not separated are; those are
 * enumerated over their offsets.  Exact whenever that prefix has at most 2^22
 * elements (any layout of at most 2^22 elements, and any larger one whose big
 * leaves are separated,
 * e.g. (3,2,M):(2,3,8) for every M); beyond that *result 0 means not proven
 * injective.  A stride-0 leaf of extent > 1 is not injective.  A swizzle never
 * changes the answer. */
int lr_is_injective(const lr_layout* L, int32_t* result);

/* Widest vector (in elements, a power of two with elems*elem_bytes <= 16) that a
 * copy from src to dst can move as one unit, assuming 16-byte-aligned buffers
 * ([CuTe algebra page, section 2.3]: the common part of the two inverse layouts
 * gives the widest contiguous copy).  Computed from the joint flat form: the
 * extent of the leading mode with stride 1 on both sides, limited so that every
 * other stride and each swizzle's M keep the vectors aligned.  1 when dst is not
 * injective or no joint form exists. */
int lr_max_common_vector(const lr_layout* src, const lr_layout* dst, size_t elem_bytes, int64_t* elems);

/* Thread maps as layouts over the thread id.  [ThreadMap page, section 2.2]:
 * strip-mined offset(tid) = tid%P + ((tid/P)%S)*kRow + (tid/(P*S))*(P*S*kRow),
 * i.e. the layout (P, S, ceil(T/(P*S))):(1, kRow, P*S*kRow).  strips == 0 gives
 * the base pitch-linear map of [ThreadMap page, section 1.2], offset =
 * tid%P + (tid/P)*kRow, i.e. (P, ceil(T/P)):(1, kRow). */
int lr_thread_map(int64_t pitch, int64_t strips, int64_t krow, int64_t threads, lr_layout* out);

/* --------------------------------------------------------------- inspection */

/* Print a layout with two top-level modes as a grid ([print_layout page, sections
 * 2.3 and 3.1]: rows walk mode 0, columns walk mode 1, each cell is the offset of
 * (row, col)).  First line: the text form of L.  Cells are right-aligned to the
 * widest offset ([print_layout page, section 6.3]) and separated by one space;
 * every line ends in '\n'.  *needed (if needed != NULL) receives the bytes the text
 * takes with its NUL, also when buf is NULL or cap too small (LR_ERR_CAPACITY,
 * buf untouched).  LR_ERR_INVALID unless L has exactly two top-level modes and at
 * most 2^20 cells. */
int lr_layout_print(const lr_layout* L, char* buf, size_t cap, size_t* needed);

/* Thread-to-offset table ([ThreadMap page, section 5.3]): for t = 0..n-1 the line
 * "thread <t> -> offset <L(t)>\n", both numbers right-aligned to the widest.
 * 1 <= n <= min(size(L), 2^20) (LR_ERR_INVALID otherwise); buf, cap and needed as
 * lr_layout_print. */
int lr_layout_print_table(const lr_layout* L, int64_t n, char* buf, size_t cap, size_t* needed);

#define LR_WAVE_LANES 64

/* Result of lr_access_check: lane t of one wavefront accesses the elem_bytes bytes
 * at element offset L(t). */
typedef struct {
  int32_t lanes, elem_bytes;  /* as passed */
  int32_t banks;              /* LDS banks of 4 bytes in the model used */
  int32_t lanes_per_phase;    /* lanes served together in the model used */
  int32_t line_bytes;         /* cache-line size used for `lines` */
  int32_t phases;             /* ceil(lanes / lanes_per_phase) */
  int32_t cycles;             /* sum over phases of the phase's worst bank ways */
  int32_t conflict_cycles;    /* cycles - phases; 0 means conflict-free */
  int32_t ways_max;           /* worst ways in any phase (1 = conflict-free) */
  int32_t bank_words[LR_WAVE_LANES]; /* distinct words per bank in the first worst phase */
  int32_t adjacent;           /* 1 if L(t+1) == L(t) + 1 for every t < lanes-1 */
  int32_t first_gap;          /* smallest t with L(t+1) != L(t) + 1, else -1 */
  int64_t lines;              /* distinct line_bytes-byte lines the lanes touch */
  int64_t min_lines;          /* ceil(distinct bytes touched / line_bytes) */
  int64_t offsets[LR_WAVE_LANES]; /* L(t) for t < lanes, in elements */
} lr_access_report;

/* LDS models for lr_access_check. */
#define LR_LDS_CUSTOM 0       /* banks and lanes_per_phase as passed */
#define LR_LDS_GFX950_READ 1  /* gfx950 ds_read: elem_bytes <= 4: 32 banks, 32 lanes a phase;
                                 8: 64 banks, 32 lanes; 16: 64 banks, 16 lanes */
#define LR_LDS_GFX950_WRITE 2 /* gfx950 ds_write: elem_bytes <= 4: 32 banks, 32 lanes a phase;
                                 8: 32 banks, 16 lanes; 16: 32 banks, 8 lanes */

/* The two checks the print_layout page (section 6.4) asks of a candidate layout,
 * for lanes 0..lanes-1 of one wavefront accessing L(0..lanes-1): whether adjacent
 * lanes hit adjacent offsets, and how evenly the lanes spread over the LDS banks
 * ([print_layout page, sections 4.3 and 5.2]: distinct 4-byte words in one bank are
 * served one after another, one word read by several lanes is served once).  Lanes
 * are served in phases of lanes_per_phase consecutive lanes, a phase taking as many
 * cycles as its busiest bank has distinct words.  lds_model LR_LDS_GFX950_READ or
 * LR_LDS_GFX950_WRITE takes banks and lanes_per_phase from the measured gfx950
 * behaviour (pass 0 for both); LR_LDS_CUSTOM uses them as given, each in [1, 64]
 * (banks = lanes_per_phase = lanes = 32 is the page's warp model).  line_bytes 0
 * means 128.  lanes in [1, min(64, size(L))] (LR_ERR_INVALID otherwise),
 * elem_bytes as lr_layout_copy (LR_ERR_ELEM_BYTES); LR_ERR_OVERFLOW if a byte
 * address does not fit in int64. */
int lr_access_check(const lr_layout* L, size_t elem_bytes, int32_t lanes, int32_t lds_model, int32_t banks,
                    int32_t lanes_per_phase, int32_t line_bytes, lr_access_report* out);

/* --------------------------------------------------------------- copy plan */

/* Copy paths (what lr_copy_plan chose). */
typedef enum {
  LR_PATH_GENERIC = 0,    /* one unit (vec_elems elements) per lane over the joint modes */
  LR_PATH_VECTOR = 1,     /* same kernel, 16-byte units along the common contiguous mode */
  LR_PATH_TRANSPOSE = 2,  /* register-blocked tile transpose, tiles staged in LDS */
  LR_PATH_INTERLEAVE = 3, /* narrow dst-contiguous mode (<= 16 bytes) interleaved in registers */
  LR_PATH_STAGED = 4,     /* compact source footprint per tile staged in LDS, gathered */
  LR_PATH_DUAL = 5,       /* no joint refinement: each side evaluated from the index */
  LR_PATH_ALIAS = 6,      /* non-injective dst, sequential last-writer semantics */
  LR_PATH_TRANSPOSE_DIRECT = 7, /* register-blocked transpose storing straight to global */
  LR_PATH_DEINTERLEAVE = 8,    /* short src-contiguous mode (2..8 channels, <= 16 bytes) spread
                                  into planes: the mirror of the interleave */
  LR_PATH_BATCHED = 9          /* a batch of small matrices, each compact on both sides (up to
                                  8 KiB, sides multiples of a 16-byte chunk): whole matrices per
                                  wavefront staged in LDS, transposed in registers */
} lr_path;

/* Copy flags. */
#define LR_COPY_ORDERED_ALIAS 0x1u   /* allow a non-injective dst: result equals the sequential
                                        loop over k = 0..N-1, so the greatest k wins */
#define LR_COPY_WIDE_INDEX 0x2u      /* force 64-bit index arithmetic (generic/dual paths only) */
#define LR_COPY_FORCE_PATH(p) ((((uint32_t)(p)) + 1u) << 8) /* force an lr_path; LR_ERR_PATH if it
                                                              does not apply */

typedef struct {
  int32_t path;        /* lr_path */
  int32_t elem_bytes;  /* bytes per element after fusing the common contiguous prefix */
  int32_t vec_elems;   /* elements (of elem_bytes) per lane unit or per register-block row */
  int32_t wide;        /* 1 if 64-bit index arithmetic is used */
  int32_t joint_rank;  /* number of joint modes (0 for the dual/alias paths) */
  int32_t a_mode;      /* joint mode contiguous in src (transpose/interleave), else -1 */
  int32_t b_mode;      /* joint mode contiguous in dst (transpose/interleave), else -1 */
  int32_t b2_mode;     /* transpose: mode continuing b_mode in dst, grouped with it, else -1 */
  int32_t block;       /* threads per workgroup */
  int32_t streaming;   /* 1 if stores (and loads, see load_policy) are non-temporal: by
                          default when the source plus destination bytes reach 64 MiB, a
                          quarter of the 256 MiB last-level cache, except for element tiles
                          (transposes of rows without aligned 16-byte chunks), which keep
                          ordinary accesses at any size, and the element-granular channel
                          shuffle (planes without aligned chunks), which streams from 256 MiB */
  int32_t order;       /* transpose: workgroup -> tile order (0 a-tiles fastest, 1 b-tiles
                          fastest, 2 diagonal with a fastest, 3 diagonal over 4 x 4 tile groups,
                          4 diagonal with b fastest; 5..9 the same over workgroup numbers
                          grouped by XCD, each XCD taking a contiguous run); -1 on other paths */
  int32_t direct;      /* 1 if the source tile goes straight from global memory into LDS
                          (staged and transpose paths) */
  int32_t load_policy;  /* cache-policy bits of the source loads: 0 plain, 2 non-temporal */
  int32_t store_policy; /* of the destination stores: 0 plain, 2 non-temporal, 18 non-temporal
                           with the sc1 scope bit (streaming 16-byte stores issued as buffer
                           stores: the LDS transpose when a tile's destination span is under
                           4 GiB; the vector path, the narrow interleave and the channel
                           shuffle when the destination's is) */
  int32_t vector_order; /* vector/generic: traversal after the common contiguous mode (0
                           destination order, 1 source order, 2 source order in blocks of
                           destination runs, 3 tiles of atoms through LDS: a_mode continues
                           the common mode in the source, b_mode in the destination, tiles of
                           tile_a x tile_b atoms); -1 on other paths */
  int32_t gather_chunks; /* staged: destination chunks of one tile per 32-lane slice of the
                            gather (a slice covers 32 / gather_chunks tiles); -1 elsewhere */
  int32_t pipeline_tiles; /* transpose: tiles per workgroup of the pipelined kernel, 0 when it
                             is not used */
  int32_t transpose_reads; /* LDS transpose: 1 when the tile is read with the gfx950 transpose
                              reads (ds_read_b64_tr_b16, ds_read_b64_tr_b8), 0 otherwise */
  int32_t batch_matrices;  /* batched: whole matrices per wavefront; -1 on other paths */
  int32_t batch_swizzle[6]; /* batched: the LDS slot of 16-byte chunk c of a wavefront's region
                               is c ^ (((c >> [0]) & [1]) << [2]) ^ (((c >> [3]) & [4]) << [5]) */
  int32_t batch_order;     /* batched: blocks of a matrix over lanes, 0 a-blocks fastest, 1
                              b-blocks fastest; -1 on other paths */
  int64_t tile_a, tile_b; /* tile extents in the a/b modes (transpose), tiles per block (staged),
                             the matrix (batched) */
  int64_t grid;        /* workgroups launched */
  int64_t n_elems;     /* logical elements of the original layouts */
  int64_t blocks;      /* launches: 1, or the number of blocks a copy too large for 32-bit offsets
                          is cut into (each planned on its own; the fields above then describe
                          the first block, joint modes excepted) */
  int64_t ext[2 * LR_MAX_LEAVES];   /* joint modes, sorted by dst stride, in fused elements */
  int64_t s_src[2 * LR_MAX_LEAVES];
  int64_t s_dst[2 * LR_MAX_LEAVES];
} lr_plan;

/* Plan a copy without launching anything (host only).  Checks everything
 * lr_layout_copy checks.  src_align/dst_align are the byte alignments of the
 * buffers (pass 16 for "aligned"). */
int lr_copy_plan(const lr_layout* Ls, int64_t src_capacity_elems, size_t src_align,
                 const lr_layout* Ld, int64_t dst_capacity_elems, size_t dst_align,
                 size_t elem_bytes, uint32_t flags, lr_plan* out);

/* Overrides of the planner's launch choices, for measurement and tests.  A field
 * of -1 leaves the choice to the planner (lr_copy_tuning_init sets every field to
 * -1); any other value is used where the chosen path has that knob and ignored
 * elsewhere.  No override changes what is copied, only how: every combination the
 * planner accepts gives the same destination bytes.  A value the path cannot honour
 * (a tile shape whose exchange does not fit the LDS, say) falls back to the
 * planner's choice; a value outside the listed range gives LR_ERR_INVALID. */
typedef struct {
  int32_t load_policy;     /* 0 plain loads, 2 non-temporal */
  int32_t store_policy;    /* 0 plain stores, 2 non-temporal, 18 non-temporal with the sc1 scope
                              bit where the kernel issues buffer stores (else as 2).  A load
                              policy different from the store policy is available on the
                              generic and vector paths only (elsewhere: LR_ERR_PATH) */
  int32_t units_per_lane;  /* generic/vector: 1 or 4 */
  int32_t vector_order;    /* vector: modes after the common contiguous one walked in 0
                              destination order, 1 source order, 2 source order in blocks
                              of destination runs, 3 tiles of atoms through LDS where the
                              common mode is an atom of 32-256 bytes, or of up to 512 bytes
                              that are not whole 128-byte lines, that different modes
                              continue in the source and the destination (else 1; see
                              lr_plan.vector_order) */
  int32_t interleave_form; /* interleave: 0 one chunk per lane per head, 1 one destination
                              chunk per lane from narrow loads, 2 the channel shuffle */
  int32_t tile_shape;      /* transpose: 0..8, the tile shapes of lr_plan.tile_a/tile_b (16-byte
                              chunks a x b: 16x16, 32x16, 16x32, 32x32, 32x8, 64x8, 64x16, 8x8,
                              8x32) */
  int32_t tile_order;      /* transpose: 0..9, as lr_plan.order (5..9 not with pipeline_tiles) */
  int32_t element_tiles;   /* transpose: 0 chunk tiles, 1 element-granular tiles */
  int32_t direct_loads;    /* staged and LDS transpose: 0 through registers, 1 global -> LDS */
  int32_t gather_chunks;   /* staged: destination chunks of one tile per 32-lane slice of
                              the gather (1, 2, 4, 8, 16 or 32; see lr_plan.gather_chunks) */
  int32_t pipeline_tiles;  /* LDS transpose with 16-byte chunks in tile shapes 0-2: 0 one tile
                              per workgroup; 2..64 that many tiles per workgroup, software-
                              pipelined through two LDS tiles with direct loads (the next tile's
                              loads in flight while the current one is stored) */
  int32_t transpose_reads; /* LDS transpose with direct loads (or pipelined), 2- or 1-byte
                              elements in 16-byte chunks, tile shapes 0-3: 0 each lane reads V
                              whole LDS rows and transposes them in registers; 1 the gfx950
                              transpose reads (ds_read_b64_tr_b16, ds_read_b64_tr_b8) hand each
                              lane one column of four (eight) rows.  For 1-byte elements it
                              implies 16-byte chunks unless chunk_bytes is 8 */
  int32_t chunk_bytes;     /* transpose of 1-byte elements: 8 or 16 bytes per chunk (the most
                              the layout's strides and alignment allow) */
  int32_t batch_swizzle;   /* batched: 0..15, the LDS swizzle of that index in the planner's
                              candidate list (lr_plan.batch_swizzle shows it) */
  int32_t batch_order;     /* batched: 0 a-blocks fastest over lanes, 1 b-blocks fastest */
  int32_t workgroup_lanes; /* vector/generic path with one 16-byte or narrower unit per lane (not
                              64-bit indices) and its tiles of atoms, the interleave with one
                              destination chunk per lane, the channel shuffle (both
                              directions, chunk form) and the staged gather (raised to the
                              16-byte destination chunks of one tile where that is more):
                              64, 128 or 256 lanes per workgroup */
  int32_t transpose_blocks; /* LDS transpose through registers (not direct loads), 16-byte chunks
                              (8-byte for 1-byte elements), tile shapes other than 7 (an even b
                              side and at least a wavefront's worth of lanes):
                              1 one V x V register block per lane, 2 two blocks per lane (half
                              the workgroup's lanes for the same tile) */
} lr_copy_tuning;

/* Every field of *t to -1 (the planner's choices). */
void lr_copy_tuning_init(lr_copy_tuning* t);

/* lr_copy_plan / lr_layout_copy with overrides; tuning == NULL is the same as
 * lr_copy_plan / lr_layout_copy. */
int lr_copy_plan_tuned(const lr_layout* Ls, int64_t src_capacity_elems, size_t src_align,
                       const lr_layout* Ld, int64_t dst_capacity_elems, size_t dst_align,
                       size_t elem_bytes, uint32_t flags, const lr_copy_tuning* tuning, lr_plan* out);

/* --------------------------------------------------------------- device */

/* Evaluate L at n 1-D indices on the GPU ([print_layout page, sections 2.3 and
 * 3.1]: the layout called on each coordinate gives its offset).  idx: device
 * int64[n], or NULL for 0..n-1.  offsets: device int64[n].  An index outside
 * [0, size) yields offset -1.  Division by the extents uses precomputed
 * multiply-high constants when size < 2^31. */
int lr_layout_eval(const lr_layout* L, const int64_t* idx, int64_t n, int64_t* offsets, void* stream);

/* Evaluate L at n coordinates on the GPU.  coords: device int64[n][ncols],
 * row-major.  ncols == nmodes: one integer per top-level mode, split
 * colexicographically inside that mode ([print_layout page, section 6.3]: a
 * layout takes integers or coordinate objects); ncols == nleaves: the natural
 * coordinate, one per leaf.  A coordinate out of range yields -1. */
int lr_layout_eval_coords(const lr_layout* L, const int64_t* coords, int64_t n, int32_t ncols,
                          int64_t* offsets, void* stream);

/* The layout-remapping copy: for every logical index k of [0, N),
 *   dst[Ld(k)] = src[Ls(k)]      (elem_bytes bytes each, bitwise)
 * ([CuTe algebra page, sections 2.3 and 5.1]: a copy between two layouts that
 * differ only in arrangement).  Elements of dst outside the image of Ld are not
 * written.  src/dst: device pointers; capacities in elements bound cosize of each
 * layout (LR_ERR_BOUNDS).  size(Ls) must equal size(Ld) (LR_ERR_SIZE_MISMATCH,
 * the runtime form of [CuTe algebra page, section 3.3]'s compatibility check).
 * The byte ranges [src, src+cap*eb) and [dst, dst+cap*eb) must not overlap
 * (LR_ERR_OVERLAP).  A non-injective Ld needs LR_COPY_ORDERED_ALIAS
 * (LR_ERR_ALIAS otherwise); the ordered copy then handles destination cosize up
 * to 2^26 elements with N * ceil(cosize/16384) <= 2^36.  A copy whose size or
 * offsets reach 2^31 runs as blocks of its joint modes that each fit 32-bit
 * offsets, launched one after another on the stream at offset base pointers (any
 * partition is the same copy when Ld is injective); with LR_COPY_WIDE_INDEX, a
 * swizzle, a forced path or an aliased Ld it is one launch with 64-bit indices.
 * Every block is planned and checked before its launch; an error in a later block
 * (in practice only LR_ERR_HIP) returns after the earlier blocks were launched, so
 * dst is then partly written. */
int lr_layout_copy(const void* src, const lr_layout* Ls, int64_t src_capacity_elems,
                   void* dst, const lr_layout* Ld, int64_t dst_capacity_elems,
                   size_t elem_bytes, uint32_t flags, void* stream);

int lr_layout_copy_tuned(const void* src, const lr_layout* Ls, int64_t src_capacity_elems,
                         void* dst, const lr_layout* Ld, int64_t dst_capacity_elems,
                         size_t elem_bytes, uint32_t flags, const lr_copy_tuning* tuning, void* stream);

/* Debugging aid (the write-race check of an injective copy): lr_layout_copy_tuned
 * that also counts, for every destination element, the stores the kernels make to
 * it.  counts: device int32[dst_capacity_elems], owned and zeroed by the caller;
 * each store of n elements atomically adds 1 to each of their counters.  The copy
 * itself is the same launch configuration and gives the same bytes.  A correct
 * copy leaves 1 at every offset in the image of Ld and 0 elsewhere -- also for an
 * aliased Ld under LR_COPY_ORDERED_ALIAS, where only the last writer of each
 * offset stores ([CuTe algebra page, section 2.3]: the copy moves each element
 * from its source offset to its destination offset).  Slow: meant for tests.
 * LR_ERR_INVALID if counts is NULL; every other error as lr_layout_copy. */
int lr_layout_copy_count_writes(const void* src, const lr_layout* Ls, int64_t src_capacity_elems,
                                void* dst, const lr_layout* Ld, int64_t dst_capacity_elems,
                                size_t elem_bytes, uint32_t flags, const lr_copy_tuning* tuning,
                                int32_t* counts, void* stream);

/* ------------------------------------------------------------------ misc */

/* Static text for a status code. */
const char* lr_strerror(int code);

/* Text of the last HIP error seen by an lr_* call on this thread ("" if none). */
const char* lr_last_hip_error(void);

/* Library version, e.g. "0.1.0". */
const char* lr_version(void);

#if defined(__GNUC__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* LAYOUT_REMAP_H */
