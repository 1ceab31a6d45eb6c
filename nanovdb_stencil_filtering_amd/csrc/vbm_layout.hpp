// Blob layout of a built grid (include/vbm.h documents every section): the
// header fields and 256-byte aligned section offsets that follow from the
// counts.  Shared by the host builder and the device-side builder so that both
// produce the same bytes.
#pragma once

#include <stdint.h>

#include <cstring>

#include "vbm.h"

namespace vbm_layout {

constexpr uint64_t kAlign = 256;
constexpr uint64_t kMaxActive = 0xFFFFFFFEull;  // indices 1..N fit in 32 bits, 0 = inactive
constexpr uint64_t kLeafBytes = 128;
constexpr uint64_t kRootBytes = 16;
constexpr uint64_t kUpperEntries = 32768;
constexpr uint64_t kLowerEntries = 4096;

inline uint64_t align_up(uint64_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

// Fills *g for a grid of n_active voxels in n_leaves leaves, n_root root tiles
// (one upper node each) and n_lower lower nodes at BlockWidth 2^log2_width.
// Returns VBM_ERR_SIZE when a count exceeds the 32-bit ids of the layout.
inline int layout(uint64_t n_active, uint64_t n_leaves, uint64_t n_root, uint64_t n_lower, int log2_width,
                  vbm_grid* g) {
  if (n_active > kMaxActive) return VBM_ERR_SIZE;
  const uint64_t W = uint64_t(1) << log2_width;
  const uint64_t words = W / 64;
  const uint64_t nb = (n_active + W - 1) / W;
  if (nb > 0xFFFFFFFFull || n_leaves > 0xFFFFFFFFull || n_root > 0xFFFFFFFFull || n_lower > 0xFFFFFFFFull)
    return VBM_ERR_SIZE;
  std::memset(g, 0, sizeof(*g));
  g->magic = VBM_GRID_MAGIC;
  g->log2_width = log2_width;
  g->n_active = n_active;
  g->n_leaves = uint32_t(n_leaves);
  g->n_blocks = uint32_t(nb);
  g->n_root = uint32_t(n_root);
  g->n_upper = uint32_t(n_root);
  g->n_lower = uint32_t(n_lower);
  uint64_t off = 0;
  g->off_leaves = off;            off = align_up(off + n_leaves * kLeafBytes);
  g->off_root = off;              off = align_up(off + n_root * kRootBytes);
  g->off_upper = off;             off = align_up(off + n_root * kUpperEntries * 4);
  g->off_lower = off;             off = align_up(off + n_lower * kLowerEntries * 4);
  g->off_block_first_leaf = off;  off = align_up(off + nb * 4);
  g->off_block_jump = off;        off = align_up(off + nb * words * 8);
  g->blob_bytes = off > 0 ? off : kAlign;
  return VBM_OK;
}

}  // namespace vbm_layout
