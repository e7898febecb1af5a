// Internal (non-ABI) declarations shared by the host algebra, the copy planner
// and the HIP launch code.  Nothing here crosses the C ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "layout_remap.h"

namespace lr {

constexpr int kMaxJoint = 2 * LR_MAX_LEAVES;  // a joint refinement has < 2*16 modes
constexpr int kMaxKernelModes = 16;           // modes a kernel argument block carries

struct Leaf {
  int64_t n, d;
};

// Checked int64 arithmetic.
inline bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }
inline bool add_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_add_overflow(a, b, r); }

int validate(const lr_layout* L);
int64_t size_of(const lr_layout* L);            // valid L only
int64_t max_linear_offset(const lr_layout* L);  // valid L only, unswizzled
int64_t cosize_bound(const lr_layout* L);       // valid L only
bool injective(const lr_layout* L);             // valid L only; exact within the limits below

// Limit of the exact injectivity check: the leaves that are not separated by
// stride (see injective) are enumerated when their combined extent stays within
// it; beyond it the answer is "not proven injective".
constexpr int64_t kExactInjectiveElems = int64_t(1) << 22;

// Multiply-high division by an invariant divisor d (1 <= d < 2^31), exact for
// dividends x < 2^31 (Granlund & Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, the round-up variant):  with l = ceil(log2 d) and
// m = ceil(2^(31+l) / d) < 2^32,  x / d == (x * m) >> (31 + l).  On the device this
// is umulhi(x, m) >> (l - 1).  d == 1 is encoded as m == 0 (quotient = x).
struct FastDiv {
  uint32_t m, s;
};
FastDiv make_fastdiv(uint32_t d);

struct JMode {
  int64_t ext, ss, sd;
};

// Joint flat form of a pair of layouts (unswizzled parts) over one index space;
// false when the two prefix-product sequences do not form one divisibility chain.
bool joint_flat(const lr_layout* s, const lr_layout* d, JMode* out, int* rank, bool sort_by_dst);

struct Swz {
  int32_t b, m, s;  // b == 0: none
};

// Transpose tile shapes in 16-byte chunks along a (source-contiguous) x b
// (destination-contiguous); the workgroup has TA * TB lanes.
constexpr int kTileShapes = 9;
constexpr int kTileTA[kTileShapes] = {16, 32, 16, 32, 32, 64, 64, 8, 8};
constexpr int kTileTB[kTileShapes] = {16, 16, 32, 32, 8, 8, 16, 8, 32};
// LDS bytes of a tile shape's exchange with V-element 16-byte chunks: TA*V rows of
// TB chunks; a shape is usable when it fits the 160 KiB of a CU.
constexpr bool shape_fits(int shape, int V) { return kTileTA[shape] * V * kTileTB[shape] * 16 <= 160 * 1024; }
// The pipelined transpose holds two tiles of shapes 0-2 (16 or 32 chunks along a, at
// least 16 along b) in LDS.
constexpr bool pipe_fits(int shape, int V) {
  return shape >= 0 && shape <= 2 && 2 * kTileTA[shape] * V * kTileTB[shape] * 16 <= 160 * 1024;
}

// Vector path, tiles of atoms (vector order 3): atoms of K = 2..32 16-byte chunks
// per tile side -- 16 up to 64-byte atoms, 8 up to 240 bytes, 4 from 256 bytes (runs
// of 512 bytes to 2 KiB).
constexpr int64_t atom_tile(int64_t K) { return K <= 4 ? 16 : (K < 16 ? 8 : 4); }

// Everything the launch code needs.
struct Plan {
  int path;           // lr_path
  int eb;             // bytes per (fused) element
  int orig_eb;        // the caller's elem_bytes
  int v;              // elements per unit (generic/vector) or per chunk (transpose/interleave)
  bool wide;
  int rank;           // joint modes (after fusion)
  JMode m[kMaxJoint];
  int a, b;           // src-contiguous / dst-contiguous modes, -1 if none
  int b2;             // transpose: mode continuing b in dst (b grouped with it), -1 if none
  Swz sw_s, sw_d;     // swizzles in units of (fused) elements
  int block;
  int64_t tile_a, tile_b;
  int64_t grid;
  int64_t n;          // logical elements (original)
  int64_t n_units;    // generic/vector: units to move
  // staged path
  int staged_inner;   // number of inner modes [0, staged_inner)
  int64_t staged_P, staged_F, staged_Fc, staged_K, staged_cpt;
  int64_t staged_cps;  // gather: destination chunks of one tile per 32-lane slice (a power
                       // of two dividing cpt); a slice of 32 lanes covers 32/cps tiles
  // alias path
  int64_t alias_windows;
  // tuning: non-temporal loads and stores (streaming data), and the transpose's
  // workgroup order (0: a-tiles fastest, 1: b-tiles fastest, 2: diagonal with a
  // fastest, 3: diagonal over 4x4 tile groups, 4: diagonal with b fastest)
  bool nt;           // non-temporal stores (and loads, except on the generic kernel)
  bool nt_ld;        // non-temporal loads
  bool policy_set;   // the caller chose the load or store policy
  int vorder;        // vector/generic: traversal order after the common mode (3: tiles of
                     // atoms through LDS, modes a and b, tile_a = tile_b atoms), -1 elsewhere
  bool direct;        // staged: direct global -> LDS loads (no register round trip)
  bool tel;           // transpose: element-granular tiles (rows without aligned chunks)
  bool twin;          // element tiles with 16-byte accesses inside each row (no swizzles,
                      // element-aligned buffers)
  bool bufst;         // streaming 16-byte stores as buffer stores with the nt and sc1 bits:
                      // vector path (destination span < 4 GiB) and LDS transpose (tile span)
  uint32_t torder;
  int unroll;         // generic/vector: units per lane (1 or 4; 4 when wide)
  int tshape;         // transpose tile shape index into kTileTA / kTileTB
  int pipe;           // pipelined transpose: tiles per workgroup (0: one tile, not pipelined)
  bool tr;            // LDS transpose: the tile is read with gfx950 transpose reads
  int tblocks;        // LDS transpose through registers: V x V blocks per lane (2, else 1)
  int64_t tiles_total; // transpose: tiles over all batch indices
  // batched small matrices: whole matrices per wavefront, matrices, the LDS chunk
  // swizzle (two XOR terms of shift, mask, target shift) and the block order (0:
  // a-blocks fastest)
  int64_t bt_mpw, bt_count;
  int bt_sw[6];
  int bt_order;
  int inarrow;        // interleave: 1 = one 16-byte store per lane from NB narrow loads,
                      // 0 = NB wide loads and stores per lane, 2 = channel shuffle through LDS,
                      // 3 = its element-granular form
};

// Channel-shuffle kernels (pixels with C interleaved channels <-> C planes) exist
// for 2..8 channels of one 16-byte chunk or less per pixel.
constexpr bool chan_supported(int eb, int64_t c) { return c >= 2 && c <= 8 && c * eb <= 16; }

// Pixels per workgroup of the element-granular channel shuffle: 16/eb per lane.
constexpr int chan_el_pixels(int eb) { return 256 * (16 / eb); }

// Plans a copy; fills `p`.  tuning may be NULL (the planner's choices).  Returns 0
// or an lr_status.
int plan_copy(const lr_layout* Ls, int64_t src_cap, size_t src_align, const lr_layout* Ld,
              int64_t dst_cap, size_t dst_align, size_t elem_bytes, uint32_t flags, const lr_copy_tuning* tuning,
              Plan* p);

// Re-checks the invariants the chosen kernel relies on; LR_ERR_PATH if violated.
int verify_plan(const Plan& p, int64_t src_cap, int64_t dst_cap);

// A copy that needs 64-bit offsets only because of its size runs as blocks of its
// joint modes, each small enough for 32-bit offsets and planned on its own.
// block_extents: per-mode block extents (cext) and the number of blocks, or false
// when the copy is not cut (not wide, 64-bit indices requested, a forced path, a
// swizzle, or too many blocks).  make_block: the layouts of the block starting at
// the per-mode indices `start`, and its base offsets on each side (elements).
bool block_extents(const Plan& p, uint32_t flags, int64_t* cext, int64_t* nblocks);
// A block of a cut copy takes the whole copy's load and store policies.
void inherit_policy(const Plan& whole, Plan* blk);
void make_block(const Plan& p, const int64_t* cext, const int64_t* start, lr_layout* ls, lr_layout* ld,
                int64_t* src_off, int64_t* dst_off);

void set_hip_error(const char* text);

// The LDS of a gfx950 compute unit as its bank-conflict counter shows it, for one
// access of elem_bytes per lane: 4 bytes and narrower see 32 banks, 32 lanes served
// at a time, for reads and writes alike; 8-byte reads see 64 banks, 32 lanes at a
// time, 16-byte reads 64 banks, 16 lanes; 8-byte writes 32 banks, 16 lanes, and
// 16-byte writes 32 banks, 8 lanes.
void gfx950_lds_model(size_t elem_bytes, bool write, int32_t* banks, int32_t* lanes_per_phase);

// Cycles one wavefront access takes in that model: lanes 0..lanes-1 access
// elem_bytes at byte_addr[t]; each phase costs its busiest bank's distinct 4-byte
// words.  ways_max (if not NULL) receives the worst phase's ways and
// worst_bank_words (if not NULL, LR_WAVE_LANES entries) its per-bank word counts.
int32_t lds_cycles(const int64_t* byte_addr, int lanes, int64_t elem_bytes, int32_t banks, int32_t lanes_per_phase,
                   int32_t* ways_max, int32_t* worst_bank_words);

}  // namespace lr
