// Host builder of the index grid and its VoxelBlockManager metadata.
//
// Builds, from a set of integer coordinates, the flat blob the GPU kernels
// read (layout in include/vbm.h):
//   * 8^3 leaves with a 512-bit value mask, a 9-bit prefix-sum directory and
//     the index of the first active voxel (openvdb PR #2258, "What changed":
//     the decode selects inside the leaf's value mask guided by the 9-bit
//     prefix-sum directory);
//   * a root table plus two levels of internal nodes (32^3 and 16^3 children)
//     that the tree-walk resolvers descend (openvdb PR #2263, "Summary":
//     root-down tree traversal per tap);
//   * per VBM block the first leaf and the jumpMap of leaf starts
//     (openvdb PR #2263, "Built on the register-decode API").
// Indices are assigned in tree order, so a block's slots cover a few
// consecutive leaves.
//
// The sort key of a voxel packs the root tile's rank and the 36-bit position
// inside the tile: upper slot (3 x 5 bits), lower slot (3 x 4 bits), voxel
// offset (3 x 3 bits), each x-major.

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "vbm.h"
#include "vbm_layout.hpp"

namespace {

constexpr uint32_t kNone = 0xFFFFFFFFu;
constexpr int64_t kCoordLimit = int64_t(1) << 30;
constexpr uint64_t kMaxActive = vbm_layout::kMaxActive;

struct RootKey {
  int32_t x, y, z;
  bool operator==(const RootKey& o) const { return x == o.x && y == o.y && z == o.z; }
  bool operator<(const RootKey& o) const {
    if (x != o.x) return x < o.x;
    if (y != o.y) return y < o.y;
    return z < o.z;
  }
};

uint64_t root_hash_key(const RootKey& k) {
  // each component of (c >> 12) fits in 19 bits for |c| < 2^30
  const uint64_t m = (uint64_t(1) << 19) - 1;
  return ((uint64_t(uint32_t(k.x)) & m) << 38) | ((uint64_t(uint32_t(k.y)) & m) << 19) | (uint64_t(uint32_t(k.z)) & m);
}

// position of a voxel inside its root tile, in tree order
uint64_t in_tile_key(int32_t x, int32_t y, int32_t z) {
  const uint64_t ux = (uint32_t(x) >> 7) & 31, uy = (uint32_t(y) >> 7) & 31, uz = (uint32_t(z) >> 7) & 31;
  const uint64_t lx = (uint32_t(x) >> 3) & 15, ly = (uint32_t(y) >> 3) & 15, lz = (uint32_t(z) >> 3) & 15;
  const uint64_t vx = uint32_t(x) & 7, vy = uint32_t(y) & 7, vz = uint32_t(z) & 7;
  return (ux << 31) | (uy << 26) | (uz << 21) | (lx << 17) | (ly << 13) | (lz << 9) | (vx << 6) | (vy << 3) | vz;
}

struct LeafRecord {
  uint64_t mask[8];
  uint64_t prefix;
  uint64_t first;
  int32_t origin[3];
  uint32_t lower;  // parent lower node
  uint32_t upper;  // parent upper node (= root tile)
  uint32_t pad[7];
};
static_assert(sizeof(LeafRecord) == 128, "leaf record is one 128-byte line");

struct RootTileRecord {
  int32_t key[3];
  uint32_t upper;
};
static_assert(sizeof(RootTileRecord) == 16, "root tile record");
static_assert(sizeof(vbm_grid) == 96 && offsetof(vbm_grid, n_active) == 8 && offsetof(vbm_grid, blob_bytes) == 40 &&
                  offsetof(vbm_grid, off_block_jump) == 88,
              "vbm_grid layout is part of the ABI");

}  // namespace

extern "C" int vbm_build(const int32_t* ijk, int64_t n, int log2_width, vbm_grid* grid, void** host_blob) {
  if (host_blob) *host_blob = nullptr;
  if (!grid || !host_blob || n < 0 || (n > 0 && !ijk)) return VBM_ERR_ARG;
  if (log2_width < 6 || log2_width > 9) return VBM_ERR_ARG;
  for (int64_t i = 0; i < 3 * n; ++i)
    if (ijk[i] <= -kCoordLimit || ijk[i] >= kCoordLimit) return VBM_ERR_RANGE;

  try {
    // ---- root tiles: dense ranks in lexicographic order -------------------
    std::unordered_map<uint64_t, uint32_t> root_rank;
    std::vector<RootKey> roots;
    for (int64_t i = 0; i < n; ++i) {
      RootKey k{ijk[3 * i] >> 12, ijk[3 * i + 1] >> 12, ijk[3 * i + 2] >> 12};
      if (root_rank.emplace(root_hash_key(k), 0).second) roots.push_back(k);
    }
    std::sort(roots.begin(), roots.end());
    for (uint32_t r = 0; r < roots.size(); ++r) root_rank[root_hash_key(roots[r])] = r;

    // ---- tree-order keys, sorted and deduplicated --------------------------
    std::vector<uint64_t> keys(static_cast<size_t>(n));
    for (int64_t i = 0; i < n; ++i) {
      const int32_t x = ijk[3 * i], y = ijk[3 * i + 1], z = ijk[3 * i + 2];
      const uint64_t r = root_rank[root_hash_key(RootKey{x >> 12, y >> 12, z >> 12})];
      keys[size_t(i)] = (r << 36) | in_tile_key(x, y, z);
    }
    std::sort(keys.begin(), keys.end());
    keys.erase(std::unique(keys.begin(), keys.end()), keys.end());
    const uint64_t N = keys.size();
    if (N > kMaxActive) return VBM_ERR_SIZE;

    // ---- leaves: runs of equal key >> 9 ------------------------------------
    std::vector<LeafRecord> leaves;
    std::vector<uint64_t> leaf_key;  // key >> 9 of each leaf (root rank | upper | lower slot)
    for (uint64_t i = 0; i < N; ++i) {
      const uint64_t lk = keys[i] >> 9;
      if (leaf_key.empty() || leaf_key.back() != lk) {
        leaf_key.push_back(lk);
        LeafRecord rec;
        std::memset(&rec, 0, sizeof(rec));
        rec.first = i + 1;
        const RootKey& rt = roots[lk >> 27];
        const uint32_t t = uint32_t(lk & ((uint64_t(1) << 27) - 1));  // upper(15) | lower(12)
        rec.origin[0] = rt.x * 4096 + int32_t((t >> 22) & 31) * 128 + int32_t((t >> 8) & 15) * 8;
        rec.origin[1] = rt.y * 4096 + int32_t((t >> 17) & 31) * 128 + int32_t((t >> 4) & 15) * 8;
        rec.origin[2] = rt.z * 4096 + int32_t((t >> 12) & 31) * 128 + int32_t(t & 15) * 8;
        leaves.push_back(rec);
      }
      const uint32_t o = uint32_t(keys[i] & 511);
      leaves.back().mask[o >> 6] |= uint64_t(1) << (o & 63);
    }
    const uint64_t L = leaves.size();
    for (LeafRecord& rec : leaves) {
      uint64_t acc = 0, dir = 0;
      for (int w = 0; w < 7; ++w) {
        acc += uint64_t(__builtin_popcountll(rec.mask[w]));
        dir |= acc << (9 * w);
      }
      rec.prefix = dir;
    }

    // ---- internal nodes ------------------------------------------------------
    const uint64_t n_root = roots.size();
    std::vector<uint32_t> upper(n_root * 32768, kNone);
    std::vector<uint32_t> lower;
    uint64_t prev_lower_key = ~uint64_t(0);
    for (uint64_t l = 0; l < L; ++l) {
      const uint64_t lower_key = leaf_key[l] >> 12;  // root rank | upper slot
      if (lower_key != prev_lower_key) {
        prev_lower_key = lower_key;
        const uint64_t r = lower_key >> 15, uslot = lower_key & 32767;
        upper[r * 32768 + uslot] = uint32_t(lower.size() / 4096);
        lower.resize(lower.size() + 4096, kNone);
      }
      lower[lower.size() - 4096 + (leaf_key[l] & 4095)] = uint32_t(l);
      leaves[l].lower = uint32_t(lower.size() / 4096 - 1);
      leaves[l].upper = uint32_t(lower_key >> 15);
    }
    const uint64_t n_lower = lower.size() / 4096;

    // ---- VBM blocks ---------------------------------------------------------
    const uint64_t W = uint64_t(1) << log2_width;
    const uint64_t words = W / 64;
    const uint64_t nb = (N + W - 1) / W;
    if (nb > 0xFFFFFFFFull || L > 0xFFFFFFFFull) return VBM_ERR_SIZE;
    std::vector<uint32_t> block_first_leaf(nb);
    std::vector<uint64_t> block_jump(nb * words, 0);
    {
      uint64_t l = 0;  // leaf containing the current index
      for (uint64_t b = 0; b < nb; ++b) {
        const uint64_t g0 = 1 + b * W;
        while (l + 1 < L && leaves[l + 1].first <= g0) ++l;
        block_first_leaf[b] = uint32_t(l);
      }
      for (uint64_t m = 1; m < L; ++m) {
        const uint64_t s = (leaves[m].first - 1) % W;
        const uint64_t b = (leaves[m].first - 1) / W;
        if (s != 0) block_jump[b * words + s / 64] |= uint64_t(1) << (s % 64);
      }
    }

    // ---- serialise ------------------------------------------------------------
    vbm_grid g;
    const int rc = vbm_layout::layout(N, L, n_root, n_lower, log2_width, &g);
    if (rc != VBM_OK) return rc;

    uint8_t* blob = static_cast<uint8_t*>(std::calloc(1, g.blob_bytes));
    if (!blob) return VBM_ERR_NOMEM;
    if (L) std::memcpy(blob + g.off_leaves, leaves.data(), L * sizeof(LeafRecord));
    for (uint64_t r = 0; r < n_root; ++r) {
      RootTileRecord rec{{roots[r].x, roots[r].y, roots[r].z}, uint32_t(r)};
      std::memcpy(blob + g.off_root + r * sizeof(rec), &rec, sizeof(rec));
    }
    if (!upper.empty()) std::memcpy(blob + g.off_upper, upper.data(), upper.size() * 4);
    if (!lower.empty()) std::memcpy(blob + g.off_lower, lower.data(), lower.size() * 4);
    if (nb) {
      std::memcpy(blob + g.off_block_first_leaf, block_first_leaf.data(), nb * 4);
      std::memcpy(blob + g.off_block_jump, block_jump.data(), nb * words * 8);
    }
    *grid = g;
    *host_blob = blob;
    return VBM_OK;
  } catch (const std::bad_alloc&) {
    return VBM_ERR_NOMEM;
  }
}

extern "C" void vbm_free_blob(void* host_blob) { std::free(host_blob); }

extern "C" const char* vbm_strerror(int status) {
  switch (status) {
    case VBM_OK: return "ok";
    case VBM_ERR_ARG: return "invalid argument";
    case VBM_ERR_SIZE: return "grid exceeds the library's size limits";
    case VBM_ERR_ALIGN: return "float buffer is not 4-byte aligned";
    case VBM_ERR_ALIAS: return "output buffer overlaps the sidecar";
    case VBM_ERR_RANGE: return "coordinate magnitude must be below 2^30";
    case VBM_ERR_HIP: return "HIP launch failed";
    case VBM_ERR_UNSUPPORTED: return "unsupported combination of shape and flags";
    case VBM_ERR_NOMEM: return "host allocation failed";
    default: return "unknown status";
  }
}
