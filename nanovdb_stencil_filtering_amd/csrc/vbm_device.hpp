// Device-side building blocks of the VBM stencil pipeline for gfx950.
//
// Header-only, so custom consumers can be written as HIP kernels on top of
// the same decode and resolvers (tests/custom_consumer.hip is one):
//   device_grid_of         the device view of a grid (header + device blob)
//   decode_slot            slot -> (leaf, voxel offset); thread-local, in registers
//   resolve_tree           one tap by a root-down tree walk (root table in
//                          global memory, or in LDS after stage_root_table)
//   stage_neighbour_table  per-block LDS table of neighbour leaf ids (all threads)
//   stage_neighbour_records  the same table holding the neighbour leaves'
//                          records (masks, prefix directory, first index), so
//                          a tap resolves from LDS alone; the library's cached
//                          cross and axis kernels use this form
//   for_each_box[_cached]  27 taps streamed to a callback in tap order
//   compute_box[_cached]   27 taps materialised into an array
//   compute_cross[_cached] 7 taps materialised into an array
//   for_each_tap[_cached|_staged]  any shape (box, cross, 19-tap axis) streamed
//   build_bricks[_staged]  the box kernels' dense 10^3 bricks of resolved taps
//
// Sources: openvdb PR #2258 "VBM select-based inverse-map decode" ("What
// changed": rank into the jumpMap, select into the value mask guided by the
// 9-bit prefix-sum directory); openvdb PR #2263 "Alternative stencil
// resolvers for VoxelBlockManager" ("Summary": plain forms walk the tree per
// tap, Cached forms stage a per-leaf neighbour table in on-chip memory built
// by all threads, blocks spanning more than MaxCachedLeaves fall back to the
// tree walk; "Built on the register-decode API": first leaf = firstLeafID,
// spanned leaves = 1 + popcount(jumpMap)); openvdb PR #2262 "NanoVDB VBM:
// Streaming box-stencil" ("What changed": tap order (di+1)*9+(dj+1)*3+(dk+1),
// streaming callback with (tap, index), index 0 = inactive).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vbm.h"

namespace vbm {

constexpr uint32_t kNoLeaf = 0xFFFFFFFFu;
constexpr uint32_t kSentinelLeaf = 0xFFFFFFFFu;
constexpr uint32_t kSentinelOffset = 0xFFFFu;
constexpr int kMaxCachedLeaves = 16;
constexpr int kBoxTaps = 27;
constexpr int kCrossTaps = 7;

struct alignas(16) Leaf {  // 128 bytes: one cache line
  uint64_t mask[8];
  uint64_t prefix;
  uint64_t first;
  int32_t origin[3];
  uint32_t lower;  // parent lower node
  uint32_t upper;  // parent upper node
  uint32_t pad[7];
};
static_assert(sizeof(Leaf) == 128, "leaf record");
static_assert(offsetof(Leaf, prefix) == 64 && offsetof(Leaf, first) == 72, "prefix and first share a 16-byte piece");

struct RootTile {
  int32_t key[3];
  uint32_t upper;
};

// Plain pointers into the device blob; passed to kernels by value.
struct DeviceGrid {
  const Leaf* leaves;
  const RootTile* root;
  const uint32_t* upper;             // n_root * 32768 lower-node ids
  const uint32_t* lower;             // n_lower * 4096 leaf ids
  const uint32_t* block_first_leaf;  // n_blocks
  const uint64_t* block_jump;        // n_blocks * (W / 64)
  uint32_t n_active;
  uint32_t n_root;
  uint32_t n_blocks;
  int32_t log2w;
};

// The device view of a grid: the header from vbm_build (or the device build)
// and the device copy of its blob.  Host or device code.
__host__ __device__ inline DeviceGrid device_grid_of(const vbm_grid& hdr, const void* d_blob) {
  const uint8_t* base = static_cast<const uint8_t*>(d_blob);
  DeviceGrid g;
  g.leaves = reinterpret_cast<const Leaf*>(base + hdr.off_leaves);
  g.root = reinterpret_cast<const RootTile*>(base + hdr.off_root);
  g.upper = reinterpret_cast<const uint32_t*>(base + hdr.off_upper);
  g.lower = reinterpret_cast<const uint32_t*>(base + hdr.off_lower);
  g.block_first_leaf = reinterpret_cast<const uint32_t*>(base + hdr.off_block_first_leaf);
  g.block_jump = reinterpret_cast<const uint64_t*>(base + hdr.off_block_jump);
  g.n_active = uint32_t(hdr.n_active);
  g.n_root = hdr.n_root;
  g.n_blocks = hdr.n_blocks;
  g.log2w = hdr.log2_width;
  return g;
}

struct Slot {
  uint32_t leaf;    // kSentinelLeaf past the last active index
  uint32_t offset;  // voxel offset o in the leaf, kSentinelOffset past the end
};

// ---------------------------------------------------------------------------
// bit helpers
// ---------------------------------------------------------------------------

// Position of the n-th (0-based) set bit of m; requires n < popcount(m).
// gfx950 has no nth-set-bit instruction: narrow by halves using popcounts.
__device__ __forceinline__ uint32_t select_in_word(uint64_t m, uint32_t n) {
  uint32_t pos = 0;
  uint32_t v = uint32_t(m);
  uint32_t c = __popc(v);
  if (n >= c) {
    n -= c;
    v = uint32_t(m >> 32);
    pos = 32;
  }
  c = __popc(v & 0xFFFFu);
  if (n >= c) { n -= c; v >>= 16; pos += 16; }
  c = __popc(v & 0xFFu);
  if (n >= c) { n -= c; v >>= 8; pos += 8; }
  c = __popc(v & 0xFu);
  if (n >= c) { n -= c; v >>= 4; pos += 4; }
  c = __popc(v & 0x3u);
  if (n >= c) { n -= c; v >>= 2; pos += 2; }
  c = v & 1u;
  if (n >= c) pos += 1;
  return pos;
}

// 9-bit field k (0..6) of the prefix directory: active voxels in mask words
// 0..k.  Field k occupies bits 9k..9k+8 of the 64-bit directory; read with
// 32-bit operations (funnel shift across the two halves).
__device__ __forceinline__ uint32_t prefix_field(uint64_t dir, uint32_t k) {
  const uint32_t lo = uint32_t(dir), hi = uint32_t(dir >> 32);
  const uint32_t p = 9 * k;
  const uint32_t x = p < 32 ? __builtin_amdgcn_alignbit(hi, lo, p) : (hi >> (p - 32));
  return x & 511u;
}

// Index of voxel offset o in leaf L, 0 if the voxel is inactive:
// leafFirst + (active voxels in the words before o's word) + (active voxels
// below o in its word).  32-bit operations on the two halves of the word.
// R is a leaf record (Leaf) or its first 80 bytes staged in LDS (StagedLeaf).
template <class R>
__device__ __forceinline__ uint32_t index_in_leaf(const R& L, uint32_t o) {
  const uint32_t w = o >> 6, b = o & 63;
  const uint64_t m = L.mask[w];
  const uint32_t lo = uint32_t(m), hi = uint32_t(m >> 32);
  const bool upper = b >= 32;
  const uint32_t half = upper ? hi : lo;
  const uint32_t sh = b & 31;
  const uint32_t below = __builtin_amdgcn_ubfe(half, 0, sh);          // bits of the half below o
  const uint32_t rank = __popc(below) + (upper ? __popc(lo) : 0u);
  const uint32_t before = w ? prefix_field(L.prefix, w - 1) : 0u;
  const uint32_t idx = uint32_t(L.first) + before + rank;
  return ((half >> sh) & 1u) ? idx : 0u;
}

// index_in_leaf of a Leaf record in global memory with the directory and the
// first index read in one 16-byte load (they share the record's fifth 16-byte
// piece), so the lookup is two loads from the record.  The tree walks with the
// root table in LDS use this form; the arithmetic is index_in_leaf's.
__device__ __forceinline__ uint32_t index_in_leaf_16(const Leaf& L, uint32_t o) {
  const uint32_t w = o >> 6, b = o & 63;
  const uint64_t m = L.mask[w];
  const uint4 pf = *reinterpret_cast<const uint4*>(&L.prefix);  // prefix lo, prefix hi, first lo, first hi
  const uint32_t lo = uint32_t(m), hi = uint32_t(m >> 32);
  const bool upper = b >= 32;
  const uint32_t half = upper ? hi : lo;
  const uint32_t sh = b & 31;
  const uint32_t below = __builtin_amdgcn_ubfe(half, 0, sh);
  const uint32_t rank = __popc(below) + (upper ? __popc(lo) : 0u);
  const uint32_t before = w ? prefix_field(uint64_t(pf.y) << 32 | pf.x, w - 1) : 0u;
  const uint32_t idx = pf.z + before + rank;
  return ((half >> sh) & 1u) ? idx : 0u;
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------

// Number of leaves block b spans: 1 + popcount(jumpMap).
__device__ __forceinline__ uint32_t block_span(const DeviceGrid& g, uint32_t b) {
  const uint32_t words = 1u << (g.log2w - 6);
  const uint64_t* jm = g.block_jump + uint64_t(b) * words;
  uint32_t span = 1;
  for (uint32_t k = 0; k < words; ++k) span += __popcll(jm[k]);
  return span;
}

// Select stage of the decode: given the slot's leaf, the voxel's rank inside
// the leaf picks the mask word through the prefix directory (the number of
// fields <= rank), then an in-word select gives the voxel offset.
__device__ __forceinline__ Slot select_in_leaf(const DeviceGrid& g, uint32_t leaf, uint64_t idx) {
  const Leaf& L = g.leaves[leaf];
  const uint32_t r = uint32_t(idx - L.first);  // rank of the voxel inside its leaf
  const uint64_t dir = L.prefix;
  uint32_t word = 0;
#pragma unroll
  for (uint32_t k = 0; k < 7; ++k) word += prefix_field(dir, k) <= r ? 1u : 0u;
  const uint32_t before = word ? prefix_field(dir, word - 1) : 0u;
  return Slot{leaf, 64 * word + select_in_word(L.mask[word], r - before)};
}

// Set bits of the 64-bit word {hi, lo} at positions 0..b (inclusive).
__device__ __forceinline__ uint32_t rank_inclusive(uint32_t lo, uint32_t hi, uint32_t b) {
  const uint32_t sh = b & 31;
  const uint32_t keep = (2u << sh) - 1u;  // bits 0..sh (all 32 when sh == 31)
  return b < 32 ? __popc(lo & keep) : __popc(lo) + __popc(hi & keep);
}

// Inverse-map decode of slot s of block b: the leaf is firstLeafID plus the
// leaf starts (jumpMap bits) at or before s, then select_in_leaf.  O(1) per
// slot, no shared memory, divergence-safe; any slot may be passed.
__device__ __forceinline__ Slot decode_slot(const DeviceGrid& g, uint32_t b, uint32_t s) {
  const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + s;
  if (idx > g.n_active) return Slot{kSentinelLeaf, kSentinelOffset};
  const uint32_t words = 1u << (g.log2w - 6);
  const uint64_t* jm = g.block_jump + uint64_t(b) * words;
  const uint32_t wi = s >> 6;
  uint32_t rank = 0;
  for (uint32_t k = 0; k < wi; ++k) rank += __popcll(jm[k]);
  const uint64_t w = jm[wi];
  rank += rank_inclusive(uint32_t(w), uint32_t(w >> 32), s & 63);
  return select_in_leaf(g, g.block_first_leaf[b] + rank, idx);
}

// decode_slot for the calling work-item's own slot s (default threadIdx.x):
// one wave64 per 64 consecutive slots, s & 63 the lane.  The jumpMap word of
// the wave is uniform, so the rank is a scalar popcount over the earlier
// words plus the lane's rank in its wave's word (v_mbcnt over the two halves)
// plus the lane's own bit.
__device__ __forceinline__ Slot decode_own_slot(const DeviceGrid& g, uint32_t b, uint32_t s = threadIdx.x) {
  const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + s;
  const uint32_t words = 1u << (g.log2w - 6);
  const uint64_t* jm = g.block_jump + uint64_t(b) * words;
  const uint32_t wi = __builtin_amdgcn_readfirstlane(s >> 6);  // wave index in the workgroup
  uint32_t rank = 0;
  for (uint32_t k = 0; k < wi; ++k) rank += __popcll(jm[k]);
  const uint64_t w = jm[wi];
  const uint32_t lo = uint32_t(w), hi = uint32_t(w >> 32);
  const uint32_t lane = s & 63;
  rank += __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));  // bits below the lane
  rank += ((lane < 32 ? lo : hi) >> (lane & 31)) & 1u;                     // the lane's own bit
  if (idx > g.n_active) return Slot{kSentinelLeaf, kSentinelOffset};
  return select_in_leaf(g, g.block_first_leaf[b] + rank, idx);
}

// ---------------------------------------------------------------------------
// tree walk
// ---------------------------------------------------------------------------

// Leaf containing voxel (x, y, z), kNoLeaf if none: root table (binary search
// over sorted keys), then upper node, then lower node.
__device__ __forceinline__ uint32_t find_leaf(const DeviceGrid& g, int32_t x, int32_t y, int32_t z) {
  const int32_t rx = x >> 12, ry = y >> 12, rz = z >> 12;
  uint32_t lo = 0, hi = g.n_root;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    const RootTile t = g.root[mid];
    const bool less = t.key[0] < rx || (t.key[0] == rx && (t.key[1] < ry || (t.key[1] == ry && t.key[2] < rz)));
    if (less) lo = mid + 1; else hi = mid;
  }
  if (lo >= g.n_root) return kNoLeaf;
  const RootTile t = g.root[lo];
  if (t.key[0] != rx || t.key[1] != ry || t.key[2] != rz) return kNoLeaf;
  const uint32_t uslot = ((uint32_t(x) >> 7) & 31) << 10 | ((uint32_t(y) >> 7) & 31) << 5 | ((uint32_t(z) >> 7) & 31);
  const uint32_t lower = g.upper[uint64_t(t.upper) * 32768 + uslot];
  if (lower == kNoLeaf) return kNoLeaf;
  const uint32_t lslot = ((uint32_t(x) >> 3) & 15) << 8 | ((uint32_t(y) >> 3) & 15) << 4 | ((uint32_t(z) >> 3) & 15);
  return g.lower[uint64_t(lower) * 4096 + lslot];
}

// Index of voxel (x, y, z) by a root-down tree walk, 0 if inactive.
__device__ __forceinline__ uint32_t resolve_tree(const DeviceGrid& g, int32_t x, int32_t y, int32_t z) {
  const uint32_t leaf = find_leaf(g, x, y, z);
  if (leaf == kNoLeaf) return 0u;
  return index_in_leaf(g.leaves[leaf], (uint32_t(x) & 7) << 6 | (uint32_t(y) & 7) << 3 | (uint32_t(z) & 7));
}

// ---------------------------------------------------------------------------
// root table in LDS
// ---------------------------------------------------------------------------
// The search over the root keys is the first and longest link of a walk's
// chain of dependent loads (three or more steps before the upper node's
// entry).  A kernel whose taps are tree walks copies a grid's root table into
// LDS once per workgroup when it has at most kLdsRootTiles tiles, and its
// walks search that copy; a grid with more tiles is searched in global memory.
// The walk is the same root-down walk with the same answers either way.
constexpr uint32_t kLdsRootTiles = 64;  // 1 KiB

struct LdsRoot {
  const RootTile* tiles;  // the workgroup's copy, in LDS (read only when staged)
  bool staged;            // workgroup-uniform: g.n_root <= kLdsRootTiles
};

// Copies the root table into `lds` (room for kLdsRootTiles tiles, in LDS) if
// it fits.  Every thread of the workgroup calls this before its first walk;
// it ends with a barrier.
__device__ __forceinline__ LdsRoot stage_root_table(const DeviceGrid& g, RootTile* lds) {
  const bool staged = g.n_root <= kLdsRootTiles;
  if (staged)
    for (uint32_t i = threadIdx.x; i < g.n_root; i += blockDim.x) lds[i] = g.root[i];
  __syncthreads();
  return LdsRoot{lds, staged};
}

// Leaf containing voxel (x, y, z) below upper node `upper`: its upper-node
// entry, then its lower-node entry; kNoLeaf if none (the steps of find_leaf
// below the root).
__device__ __forceinline__ uint32_t leaf_below(const DeviceGrid& g, uint32_t upper, int32_t x, int32_t y, int32_t z) {
  const uint32_t uslot = ((uint32_t(x) >> 7) & 31) << 10 | ((uint32_t(y) >> 7) & 31) << 5 | ((uint32_t(z) >> 7) & 31);
  const uint32_t lower = g.upper[uint64_t(upper) * 32768 + uslot];
  if (lower == kNoLeaf) return kNoLeaf;
  const uint32_t lslot = ((uint32_t(x) >> 3) & 15) << 8 | ((uint32_t(y) >> 3) & 15) << 4 | ((uint32_t(z) >> 3) & 15);
  return g.lower[uint64_t(lower) * 4096 + lslot];
}

// resolve_tree with the root search over the LDS copy (the global one when not
// staged), by halving steps from the largest power of two not above n_root (a
// workgroup-uniform trip count): lo grows by `step` while the tile just below
// lo + step is at or below the key, so it ends as the number of tiles at or
// below (rx, ry, rz), and the last tile taken is the greatest of them: the
// voxel's tile if it is equal to the key.  That tile's fields are kept as they
// are read, so no read follows the search.
__device__ __forceinline__ uint32_t resolve_tree(const DeviceGrid& g, const LdsRoot& r, int32_t x, int32_t y,
                                                 int32_t z) {
  if (!r.staged) return resolve_tree(g, x, y, z);
  const int32_t rx = x >> 12, ry = y >> 12, rz = z >> 12;
  const uint32_t n = g.n_root;
  uint32_t lo = 0, upper = 0;
  bool equal = false;
  for (uint32_t step = n ? 1u << (31 - __builtin_clz(n)) : 0u; step; step >>= 1) {
    if (lo + step <= n) {
      const RootTile t = r.tiles[lo + step - 1];
      if (!(rx < t.key[0] || (rx == t.key[0] && (ry < t.key[1] || (ry == t.key[1] && rz < t.key[2]))))) {
        lo += step;
        equal = t.key[0] == rx && t.key[1] == ry && t.key[2] == rz;
        upper = t.upper;
      }
    }
  }
  if (!equal) return 0u;
  const uint32_t leaf = leaf_below(g, upper, x, y, z);
  if (leaf == kNoLeaf) return 0u;
  return index_in_leaf_16(g.leaves[leaf], (uint32_t(x) & 7) << 6 | (uint32_t(y) & 7) << 3 | (uint32_t(z) & 7));
}

// Leaf at offset (8 dx, 8 dy, 8 dz) from leaf L (kNoLeaf if none), found
// from L's parents: inside L's lower node it is one lower-node entry; inside
// its upper node, an upper-node entry then a lower-node entry; otherwise a
// root-down walk.  Same answer as find_leaf at the neighbour's origin.
__device__ __forceinline__ uint32_t neighbour_leaf(const DeviceGrid& g, const Leaf& L, int dx, int dy, int dz) {
  const int32_t ox = L.origin[0], oy = L.origin[1], oz = L.origin[2];
  const int32_t x = ox + 8 * dx, y = oy + 8 * dy, z = oz + 8 * dz;
  const uint32_t lslot = ((uint32_t(x) >> 3) & 15) << 8 | ((uint32_t(y) >> 3) & 15) << 4 | ((uint32_t(z) >> 3) & 15);
  if (((x ^ ox) | (y ^ oy) | (z ^ oz)) >> 7 == 0) return g.lower[uint64_t(L.lower) * 4096 + lslot];
  if (((x ^ ox) | (y ^ oy) | (z ^ oz)) >> 12 == 0) {
    const uint32_t uslot =
        ((uint32_t(x) >> 7) & 31) << 10 | ((uint32_t(y) >> 7) & 31) << 5 | ((uint32_t(z) >> 7) & 31);
    const uint32_t lower = g.upper[uint64_t(L.upper) * 32768 + uslot];
    return lower == kNoLeaf ? kNoLeaf : g.lower[uint64_t(lower) * 4096 + lslot];
  }
  return find_leaf(g, x, y, z);
}

// ---------------------------------------------------------------------------
// stencil shapes
// ---------------------------------------------------------------------------

// Box tap t = (di+1)*9 + (dj+1)*3 + (dk+1); di along x, dj along y, dk along z.
__host__ __device__ constexpr int box_di(int t) { return t / 9 - 1; }
__host__ __device__ constexpr int box_dj(int t) { return (t / 3) % 3 - 1; }
__host__ __device__ constexpr int box_dk(int t) { return t % 3 - 1; }

// Cross = the box taps with |di|+|dj|+|dk| <= 1 in ascending box order:
// -x, -y, -z, centre, +z, +y, +x.
__host__ __device__ constexpr int cross_box_tap(int j) {
  return j == 0 ? 4 : j == 1 ? 10 : j == 2 ? 12 : j == 3 ? 13 : j == 4 ? 14 : j == 5 ? 16 : 22;
}

// 19-tap axis stencil (the reach of a fifth-order WENO consumer): the centre
// and +-1..+-3 along each axis, ascending lexicographic (di, dj, dk) order;
// tap 9 is the centre.  A reach of 3 < 8 leaves the leaf in at most one axis,
// so its cached table has the 7 directions of the cross.
constexpr int kAxisTaps = 19;
__host__ __device__ constexpr int axis_di(int j) { return j < 3 ? j - 3 : j >= 16 ? j - 15 : 0; }
__host__ __device__ constexpr int axis_dj(int j) { return (j >= 3 && j < 6) ? j - 6 : (j >= 13 && j < 16) ? j - 12 : 0; }
__host__ __device__ constexpr int axis_dk(int j) { return (j >= 6 && j < 13) ? j - 9 : 0; }

// Stencil shapes: tap count, cached-table directions per leaf, offsets.
struct BoxShape {
  static constexpr int kTaps = kBoxTaps, kDirs = 27;
  static constexpr int kCentre = 13;
  __host__ __device__ static constexpr int di(int t) { return box_di(t); }
  __host__ __device__ static constexpr int dj(int t) { return box_dj(t); }
  __host__ __device__ static constexpr int dk(int t) { return box_dk(t); }
};
struct CrossShape {
  static constexpr int kTaps = kCrossTaps, kDirs = 7;
  static constexpr int kCentre = 3;
  __host__ __device__ static constexpr int di(int j) { return box_di(cross_box_tap(j)); }
  __host__ __device__ static constexpr int dj(int j) { return box_dj(cross_box_tap(j)); }
  __host__ __device__ static constexpr int dk(int j) { return box_dk(cross_box_tap(j)); }
};
struct AxisShape {
  static constexpr int kTaps = kAxisTaps, kDirs = 7;
  static constexpr int kCentre = 9;
  __host__ __device__ static constexpr int di(int j) { return axis_di(j); }
  __host__ __device__ static constexpr int dj(int j) { return axis_dj(j); }
  __host__ __device__ static constexpr int dk(int j) { return axis_dk(j); }
};

// Leaf-level direction slot of a neighbour leaf in a table with DIRS entries
// per spanned leaf.  Box: 27 directions in the same order as the box taps.
// Cross: the 7 directions of the cross taps (a one-voxel reach in one axis
// leaves the leaf in at most one axis).
template <int DIRS>
__host__ __device__ constexpr int dir_slot(int dx, int dy, int dz) {
  if (DIRS == 27) return (dx + 1) * 9 + (dy + 1) * 3 + (dz + 1);
  return dx < 0 ? 0 : dy < 0 ? 1 : dz < 0 ? 2 : dz > 0 ? 4 : dy > 0 ? 5 : dx > 0 ? 6 : 3;
}

// ---------------------------------------------------------------------------
// cached resolution: per-block LDS table of neighbour leaves
// ---------------------------------------------------------------------------

// All threads of the block cooperatively fill table[j*DIRS + dir] = leaf id of
// the neighbour of spanned leaf j (first_leaf + j) in direction dir (kNoLeaf
// if absent), then one barrier.  Must be called by every thread of the block
// with span <= kMaxCachedLeaves.
template <int DIRS>
__device__ __forceinline__ void stage_neighbour_table(const DeviceGrid& g, uint32_t first_leaf, uint32_t span,
                                                      uint32_t* table) {
  for (uint32_t e = threadIdx.x; e < span * DIRS; e += blockDim.x) {
    const uint32_t j = e / DIRS, dir = e % DIRS;
    int dx, dy, dz;
    if (DIRS == 27) {
      dx = int(dir) / 9 - 1; dy = (int(dir) / 3) % 3 - 1; dz = int(dir) % 3 - 1;
    } else {
      // cross order -x, -y, -z, centre, +z, +y, +x
      const int d = int(dir);
      const int axis = d < 3 ? d : 6 - d;  // 0 = x, 1 = y, 2 = z (3 = centre)
      const int sign = d < 3 ? -1 : (d > 3 ? 1 : 0);
      dx = axis == 0 ? sign : 0; dy = axis == 1 ? sign : 0; dz = axis == 2 ? sign : 0;
    }
    table[e] = (dx | dy | dz) ? neighbour_leaf(g, g.leaves[first_leaf + j], dx, dy, dz) : first_leaf + j;
  }
  __syncthreads();
}

// Index of the neighbour (di, dj, dk) of the voxel at local position
// (x, y, z) of spanned leaf j, through the staged table: the neighbour's leaf
// direction comes from the local coordinate leaving 0..7, its offset from the
// coordinate modulo 8.
template <int DIRS>
__device__ __forceinline__ uint32_t resolve_cached(const DeviceGrid& g, const uint32_t* table, uint32_t j,
                                                   int x, int y, int z, int di, int dj, int dk) {
  const int nx = x + di, ny = y + dj, nz = z + dk;
  const uint32_t leaf = table[j * DIRS + dir_slot<DIRS>(nx >> 3, ny >> 3, nz >> 3)];
  const uint32_t o = (uint32_t(nx) & 7) << 6 | (uint32_t(ny) & 7) << 3 | (uint32_t(nz) & 7);
  const bool ok = leaf != kNoLeaf;
  const uint32_t idx = index_in_leaf(g.leaves[ok ? leaf : 0u], o);  // leaf 0 exists when any slot is valid
  return ok ? idx : 0u;
}

// The first 80 bytes of a leaf record (mask words, prefix directory, first
// index) copied to LDS as five 16-byte pieces; zeros for an absent leaf.
struct StagedLeaf {
  uint64_t mask[8];
  uint64_t prefix;
  uint64_t first;
};
static_assert(sizeof(StagedLeaf) == 80, "staged leaf is five 16-byte pieces");

// Cached resolution with the neighbour leaves' records themselves staged in
// LDS (mask words, prefix directory, first index; zeros for an absent leaf):
// staged[j * DIRS + dir] for spanned leaf j, so a tap is LDS reads and
// popcounts, with no global load before the gather's.  All threads of the
// block; ends with a barrier.  span <= kMaxCachedLeaves.
template <int DIRS>
__device__ __forceinline__ void stage_neighbour_records(const DeviceGrid& g, uint32_t first_leaf, uint32_t span,
                                                        StagedLeaf* staged) {
  for (uint32_t e = threadIdx.x; e < span * DIRS; e += blockDim.x) {
    const uint32_t j = e / DIRS, dir = e % DIRS;
    int dx, dy, dz;
    if (DIRS == 27) {
      dx = int(dir) / 9 - 1; dy = (int(dir) / 3) % 3 - 1; dz = int(dir) % 3 - 1;
    } else {
      // cross order -x, -y, -z, centre, +z, +y, +x
      const int d = int(dir);
      const int axis = d < 3 ? d : 6 - d;  // 0 = x, 1 = y, 2 = z (3 = centre)
      const int sign = d < 3 ? -1 : (d > 3 ? 1 : 0);
      dx = axis == 0 ? sign : 0; dy = axis == 1 ? sign : 0; dz = axis == 2 ? sign : 0;
    }
    const uint32_t leaf = (dx | dy | dz) ? neighbour_leaf(g, g.leaves[first_leaf + j], dx, dy, dz) : first_leaf + j;
    const bool ok = leaf != kNoLeaf;
    const uint4* src = reinterpret_cast<const uint4*>(&g.leaves[ok ? leaf : first_leaf]);
    uint4* dst = reinterpret_cast<uint4*>(staged + e);
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const uint4 v = src[k];
      dst[k] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
}

// resolve_cached through the staged records.
template <int DIRS>
__device__ __forceinline__ uint32_t resolve_staged(const StagedLeaf* staged, uint32_t j, int x, int y, int z, int di,
                                                   int dj, int dk) {
  const int nx = x + di, ny = y + dj, nz = z + dk;
  const StagedLeaf& L = staged[j * DIRS + dir_slot<DIRS>(nx >> 3, ny >> 3, nz >> 3)];
  const uint32_t o = (uint32_t(nx) & 7) << 6 | (uint32_t(ny) & 7) << 3 | (uint32_t(nz) & 7);
  return index_in_leaf(L, o);  // an absent leaf has an empty mask: 0
}

// ---------------------------------------------------------------------------
// cached resolution, brick form: per spanned leaf, a dense 10^3 block of
// resolved taps in LDS
// ---------------------------------------------------------------------------
//
// After the neighbour-leaf table is staged, the workgroup resolves once, for
// each spanned leaf, every position of the leaf grown by one voxel on each side
// (10 x 10 x 10 positions, the union of the 27-tap stencils of its voxels).
// Entry (x+1, y+1, z+1) holds the resolved tap of local position (x, y, z),
// x, y, z in -1..8, encoded as value = index * scale, or `sentinel` when
// inactive.  A voxel at (x, y, z) then finds tap (di, dj, dk) at entry
// (x+1+di, y+1+dj, z+1+dk): 27 LDS reads at fixed offsets from one address.
// Positions are resolved one (x, y) column at a time: the column's mask byte
// and the index of its first voxel come from one mask word of the centre
// leaf (z 0..7) and of its -z / +z neighbours (z = -1, z = 8).
constexpr int kBrickEdge = 10;
constexpr int kBrickCells = kBrickEdge * kBrickEdge * kBrickEdge;

struct ColumnBits {
  uint32_t bits;  // active voxels of the column at z = 0..7 (bit z)
  uint32_t base;  // index of the column's first active voxel, if any
};

// Column (wx, y) of leaf `leaf`: mask byte ((y & 7) of word wx) and the index
// of its first voxel.  kNoLeaf gives an empty column.
__device__ __forceinline__ ColumnBits column_bits(const DeviceGrid& g, uint32_t leaf, uint32_t wx, uint32_t y8) {
  const bool ok = leaf != kNoLeaf;
  const Leaf& L = g.leaves[ok ? leaf : 0u];
  const uint64_t m = L.mask[wx];
  const uint32_t lo = uint32_t(m), hi = uint32_t(m >> 32);
  const bool upper = y8 >= 32;
  const uint32_t half = upper ? hi : lo;
  const uint32_t sh = y8 & 31;
  const uint32_t below = __popc(__builtin_amdgcn_ubfe(half, 0, sh)) + (upper ? __popc(lo) : 0u);
  const uint32_t before = wx ? prefix_field(L.prefix, wx - 1) : 0u;
  const uint32_t bits = __builtin_amdgcn_ubfe(half, sh, 8);
  return ColumnBits{ok ? bits : 0u, uint32_t(L.first) + before + below};
}


// column_bits on a staged leaf record (an absent leaf has an empty mask).
__device__ __forceinline__ ColumnBits column_bits_staged(const StagedLeaf& L, uint32_t wx, uint32_t y8) {
  const uint64_t m = L.mask[wx];
  const uint32_t lo = uint32_t(m), hi = uint32_t(m >> 32);
  const bool upper = y8 >= 32;
  const uint32_t half = upper ? hi : lo;
  const uint32_t sh = y8 & 31;
  const uint32_t below = __popc(__builtin_amdgcn_ubfe(half, 0, sh)) + (upper ? __popc(lo) : 0u);
  const uint32_t before = wx ? prefix_field(L.prefix, wx - 1) : 0u;
  return ColumnBits{__builtin_amdgcn_ubfe(half, sh, 8), uint32_t(L.first) + before + below};
}

// x range of the block's voxels in each spanned leaf, for the brick build.
// The block's slots of one leaf are consecutive and, in tree order, ascend in
// x, so the leaf's first slot in the block holds its lowest x and its last
// slot its highest.  The work-item of slot s = threadIdx.x (s < W) records
// them: xr[j] = lowest x and xr[kMaxCachedLeaves + j] = highest x of spanned
// leaf j < kMaxCachedLeaves.  A slot starts its leaf's run when s = 0 or its
// jumpMap bit is set, and ends it when s = W - 1, it holds the grid's last
// index, or bit s + 1 is set.  No barrier.
__device__ __forceinline__ void record_leaf_xrange(const DeviceGrid& g, uint32_t b, const Slot& s, uint32_t first,
                                                   uint32_t* xr) {
  if (s.leaf == kSentinelLeaf) return;
  const uint32_t j = s.leaf - first;
  if (j >= uint32_t(kMaxCachedLeaves)) return;
  const uint32_t slot = threadIdx.x, lane = slot & 63;
  const uint32_t words = 1u << (g.log2w - 6);
  const uint64_t* jm = g.block_jump + uint64_t(b) * words;
  const uint32_t wi = __builtin_amdgcn_readfirstlane(slot >> 6);  // wave index in the workgroup
  const uint64_t w = jm[wi];
  const uint32_t lo = uint32_t(w), hi = uint32_t(w >> 32);
  const uint32_t next = wi + 1 < words ? uint32_t(jm[wi + 1]) : 0u;  // bit 0 follows lane 63
  auto bit = [&](uint32_t k) {  // bit k of the wave's word, k <= 64 (32-bit shifts only)
    return k < 32 ? (lo >> k) & 1u : k < 64 ? (hi >> (k - 32)) & 1u : next & 1u;
  };
  const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + slot;
  const bool starts = slot == 0 || bit(lane);
  const bool ends = slot + 1 == (1u << g.log2w) || idx == g.n_active || bit(lane + 1);
  const uint32_t x = s.offset >> 6;
  if (starts) xr[j] = x;
  if (ends) xr[kMaxCachedLeaves + j] = x;
}

// Resolve the bricks of `count` spanned leaves whose neighbour tables are
// table[jj * 27 + dir], jj < count, into brick[jj * kBrickCells + ...].  Only
// the x planes a voxel of the block can reach are resolved: xr[jj] .. xr[jj +
// kMaxCachedLeaves] (from record_leaf_xrange) grown by one on each side; the
// other planes of a brick are left unwritten and are never read.  All threads
// of the block; ends with a barrier.
__device__ __forceinline__ void build_bricks(const DeviceGrid& g, const uint32_t* table, uint32_t count,
                                             const uint32_t* xr, uint32_t scale, uint32_t sentinel,
                                             uint32_t* brick) {
  uint32_t total = 0;
  for (uint32_t jj = 0; jj < count; ++jj) total += (xr[kMaxCachedLeaves + jj] - xr[jj] + 3) * 10;
  for (uint32_t c = threadIdx.x; c < total; c += blockDim.x) {
    // column c -> (brick jj, plane xp, row yp): bricks in order, each over its planes
    uint32_t jj = 0, rem = c, xp0 = xr[0];
    for (;;) {
      const uint32_t n = (xr[kMaxCachedLeaves + jj] - xp0 + 3) * 10;
      if (rem < n) break;
      rem -= n;
      xp0 = xr[++jj];
    }
    const uint32_t xp = xp0 + rem / 10, yp = rem % 10;  // plane xp holds x = xp - 1
    const int x = int(xp) - 1, y = int(yp) - 1;
    const int dxl = x >> 3, dyl = y >> 3;  // -1, 0, +1
    const uint32_t wx = uint32_t(x) & 7, y8 = (uint32_t(y) & 7) << 3;
    const uint32_t* trow = table + jj * 27 + (dxl + 1) * 9 + (dyl + 1) * 3;
    const ColumnBits zm = column_bits(g, trow[0], wx, y8);  // -z neighbour, its z = 7
    const ColumnBits zc = column_bits(g, trow[1], wx, y8);  // the leaf column, z = 0..7
    const ColumnBits zp = column_bits(g, trow[2], wx, y8);  // +z neighbour, its z = 0
    uint32_t* out = brick + jj * kBrickCells + xp * 100 + yp * 10;
    out[0] = ((zm.bits >> 7) & 1u) ? (zm.base + __popc(zm.bits & 0x7Fu)) * scale : sentinel;
#pragma unroll
    for (uint32_t z = 0; z < 8; ++z)
      out[1 + z] = ((zc.bits >> z) & 1u) ? (zc.base + __popc(zc.bits & ((1u << z) - 1u))) * scale : sentinel;
    out[9] = (zp.bits & 1u) ? zp.base * scale : sentinel;
  }
  __syncthreads();
}

// build_bricks over leaf records staged in LDS: staged[jj * 27 + dir] is the
// record of table entry jj * 27 + dir (see fill_table_range_staged).
__device__ __forceinline__ void build_bricks_staged(const StagedLeaf* staged, uint32_t count, const uint32_t* xr,
                                                    uint32_t scale, uint32_t sentinel, uint32_t* brick) {
  uint32_t total = 0;
  for (uint32_t jj = 0; jj < count; ++jj) total += (xr[kMaxCachedLeaves + jj] - xr[jj] + 3) * 10;
  for (uint32_t c = threadIdx.x; c < total; c += blockDim.x) {
    uint32_t jj = 0, rem = c, xp0 = xr[0];
    for (;;) {
      const uint32_t n = (xr[kMaxCachedLeaves + jj] - xp0 + 3) * 10;
      if (rem < n) break;
      rem -= n;
      xp0 = xr[++jj];
    }
    const uint32_t xp = xp0 + rem / 10, yp = rem % 10;  // plane xp holds x = xp - 1
    const int x = int(xp) - 1, y = int(yp) - 1;
    const int dxl = x >> 3, dyl = y >> 3;  // -1, 0, +1
    const uint32_t wx = uint32_t(x) & 7, y8 = (uint32_t(y) & 7) << 3;
    const StagedLeaf* row = staged + jj * 27 + (dxl + 1) * 9 + (dyl + 1) * 3;
    const ColumnBits zm = column_bits_staged(row[0], wx, y8);  // -z neighbour, its z = 7
    const ColumnBits zc = column_bits_staged(row[1], wx, y8);  // the leaf column, z = 0..7
    const ColumnBits zp = column_bits_staged(row[2], wx, y8);  // +z neighbour, its z = 0
    uint32_t* out = brick + jj * kBrickCells + xp * 100 + yp * 10;
    out[0] = ((zm.bits >> 7) & 1u) ? (zm.base + __popc(zm.bits & 0x7Fu)) * scale : sentinel;
#pragma unroll
    for (uint32_t z = 0; z < 8; ++z)
      out[1 + z] = ((zc.bits >> z) & 1u) ? (zc.base + __popc(zc.bits & ((1u << z) - 1u))) * scale : sentinel;
    out[9] = (zp.bits & 1u) ? zp.base * scale : sentinel;
  }
  __syncthreads();
}

// fill_table_range that also copies each entry's leaf record into
// staged[e] (16-byte aligned LDS), so the brick build reads the masks from
// LDS instead of gathering them from global memory column by column.
__device__ __forceinline__ void fill_table_range_staged(const DeviceGrid& g, uint32_t first, uint32_t count,
                                                        StagedLeaf* staged, uint32_t worker, uint32_t workers) {
  for (uint32_t e = worker; e < count * 27; e += workers) {
    const uint32_t j = e / 27, dir = e - j * 27;
    const int dx = int(dir) / 9 - 1, dy = (int(dir) / 3) % 3 - 1, dz = int(dir) % 3 - 1;
    const uint32_t leaf = (dx | dy | dz) ? neighbour_leaf(g, g.leaves[first + j], dx, dy, dz) : first + j;
    const bool ok = leaf != kNoLeaf;
    const uint4* src = reinterpret_cast<const uint4*>(&g.leaves[ok ? leaf : 0u]);
    uint4* dst = reinterpret_cast<uint4*>(staged + e);
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const uint4 v = src[k];
      dst[k] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// Fill the neighbour-leaf table of the `count` spanned leaves starting at
// leaf `first`, entries e = worker, worker + workers, ... (no barrier).
__device__ __forceinline__ void fill_table_range(const DeviceGrid& g, uint32_t first, uint32_t count,
                                                 uint32_t* table, uint32_t worker, uint32_t workers) {
  for (uint32_t e = worker; e < count * 27; e += workers) {
    const uint32_t j = e / 27, dir = e - j * 27;
    const int dx = int(dir) / 9 - 1, dy = (int(dir) / 3) % 3 - 1, dz = int(dir) % 3 - 1;
    table[e] = (dx | dy | dz) ? neighbour_leaf(g, g.leaves[first + j], dx, dy, dz) : first + j;
  }
}

// Stage the neighbour-leaf table of the `count` spanned leaves starting at
// leaf `first` (all threads; ends with a barrier).
__device__ __forceinline__ void stage_table_range(const DeviceGrid& g, uint32_t first, uint32_t count,
                                                  uint32_t* table) {
  fill_table_range(g, first, count, table, threadIdx.x, blockDim.x);
  __syncthreads();
}

// Address of the (-1, -1, -1) tap of the voxel at local offset o in brick jj;
// tap t of the box is at offset box_brick_offset(t) from it.
__device__ __forceinline__ const uint32_t* brick_corner(const uint32_t* brick, uint32_t jj, uint32_t o) {
  return brick + jj * kBrickCells + (o >> 6) * 100 + ((o >> 3) & 7) * 10 + (o & 7);
}
__host__ __device__ constexpr int box_brick_offset(int t) { return (t / 9) * 100 + ((t / 3) % 3) * 10 + t % 3; }

// Brick-cached box: the 27 taps streamed to f(t, value) in tap order.
template <class F>
__device__ __forceinline__ void for_each_box_brick(const uint32_t* corner, F&& f) {
#pragma unroll
  for (int t = 0; t < kBoxTaps; ++t) f(t, corner[box_brick_offset(t)]);
}

// ---------------------------------------------------------------------------
// resolvers: streamed (forEach) and materialised (compute) forms
// ---------------------------------------------------------------------------

struct VoxelCoord {
  int32_t x, y, z;
};

__device__ __forceinline__ VoxelCoord voxel_coord(const DeviceGrid& g, Slot s) {
  const Leaf& L = g.leaves[s.leaf];
  return VoxelCoord{L.origin[0] + int32_t(s.offset >> 6), L.origin[1] + int32_t((s.offset >> 3) & 7),
                    L.origin[2] + int32_t(s.offset & 7)};
}

// Plain box: tap t by a tree walk, streamed to f(t, index) in tap order.
template <class F>
__device__ __forceinline__ void for_each_box(const DeviceGrid& g, Slot s, F&& f) {
  const VoxelCoord p = voxel_coord(g, s);
#pragma unroll
  for (int t = 0; t < kBoxTaps; ++t) f(t, resolve_tree(g, p.x + box_di(t), p.y + box_dj(t), p.z + box_dk(t)));
}

template <class F>
__device__ __forceinline__ void for_each_box(const DeviceGrid& g, const LdsRoot& r, Slot s, F&& f) {
  const VoxelCoord p = voxel_coord(g, s);
#pragma unroll
  for (int t = 0; t < kBoxTaps; ++t) f(t, resolve_tree(g, r, p.x + box_di(t), p.y + box_dj(t), p.z + box_dk(t)));
}

template <class F>
__device__ __forceinline__ void for_each_box_cached(const DeviceGrid& g, const uint32_t* table, uint32_t first_leaf,
                                                    Slot s, F&& f) {
  const uint32_t j = s.leaf - first_leaf;
  const int x = int(s.offset >> 6), y = int((s.offset >> 3) & 7), z = int(s.offset & 7);
#pragma unroll
  for (int t = 0; t < kBoxTaps; ++t) f(t, resolve_cached<27>(g, table, j, x, y, z, box_di(t), box_dj(t), box_dk(t)));
}

__device__ __forceinline__ void compute_box(const DeviceGrid& g, Slot s, uint64_t (&st)[kBoxTaps]) {
  for_each_box(g, s, [&](int t, uint32_t idx) { st[t] = idx; });
}

__device__ __forceinline__ void compute_box(const DeviceGrid& g, const LdsRoot& r, Slot s, uint64_t (&st)[kBoxTaps]) {
  for_each_box(g, r, s, [&](int t, uint32_t idx) { st[t] = idx; });
}

__device__ __forceinline__ void compute_box_cached(const DeviceGrid& g, const uint32_t* table, uint32_t first_leaf,
                                                   Slot s, uint64_t (&st)[kBoxTaps]) {
  for_each_box_cached(g, table, first_leaf, s, [&](int t, uint32_t idx) { st[t] = idx; });
}

// Any shape: taps by tree walks, streamed to f(tap, index) in tap order.
template <class S, class F>
__device__ __forceinline__ void for_each_tap(const DeviceGrid& g, Slot s, F&& f) {
  const VoxelCoord p = voxel_coord(g, s);
#pragma unroll
  for (int t = 0; t < S::kTaps; ++t) f(t, resolve_tree(g, p.x + S::di(t), p.y + S::dj(t), p.z + S::dk(t)));
}

template <class S, class F>
__device__ __forceinline__ void for_each_tap(const DeviceGrid& g, const LdsRoot& r, Slot s, F&& f) {
  const VoxelCoord p = voxel_coord(g, s);
#pragma unroll
  for (int t = 0; t < S::kTaps; ++t) f(t, resolve_tree(g, r, p.x + S::di(t), p.y + S::dj(t), p.z + S::dk(t)));
}

// Any shape: taps through the staged table of neighbour leaves (S::kDirs per
// spanned leaf), streamed to f(tap, index) in tap order.
template <class S, class F>
__device__ __forceinline__ void for_each_tap_cached(const DeviceGrid& g, const uint32_t* table, uint32_t first_leaf,
                                                    Slot s, F&& f) {
  const uint32_t j = s.leaf - first_leaf;
  const int x = int(s.offset >> 6), y = int((s.offset >> 3) & 7), z = int(s.offset & 7);
#pragma unroll
  for (int t = 0; t < S::kTaps; ++t) f(t, resolve_cached<S::kDirs>(g, table, j, x, y, z, S::di(t), S::dj(t), S::dk(t)));
}

// Any shape: taps through the staged neighbour records, streamed to f(tap, index).
template <class S, class F>
__device__ __forceinline__ void for_each_tap_staged(const StagedLeaf* staged, uint32_t first_leaf, Slot s, F&& f) {
  const uint32_t j = s.leaf - first_leaf;
  const int x = int(s.offset >> 6), y = int((s.offset >> 3) & 7), z = int(s.offset & 7);
#pragma unroll
  for (int t = 0; t < S::kTaps; ++t) f(t, resolve_staged<S::kDirs>(staged, j, x, y, z, S::di(t), S::dj(t), S::dk(t)));
}

__device__ __forceinline__ void compute_cross(const DeviceGrid& g, Slot s, uint64_t (&st)[kCrossTaps]) {
  const VoxelCoord p = voxel_coord(g, s);
#pragma unroll
  for (int j = 0; j < kCrossTaps; ++j) {
    const int t = cross_box_tap(j);
    st[j] = resolve_tree(g, p.x + box_di(t), p.y + box_dj(t), p.z + box_dk(t));
  }
}

__device__ __forceinline__ void compute_cross_cached(const DeviceGrid& g, const uint32_t* table,
                                                     uint32_t first_leaf, Slot s, uint64_t (&st)[kCrossTaps]) {
  const uint32_t j = s.leaf - first_leaf;
  const int x = int(s.offset >> 6), y = int((s.offset >> 3) & 7), z = int(s.offset & 7);
#pragma unroll
  for (int k = 0; k < kCrossTaps; ++k) {
    const int t = cross_box_tap(k);
    st[k] = resolve_cached<7>(g, table, j, x, y, z, box_di(t), box_dj(t), box_dk(t));
  }
}

}  // namespace vbm
