// CPU oracle for the VoxelBlockManager stencil pipeline.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
// baseline of the benchmark may load this library.  It shares no code with the
// HIP path: it rebuilds the index grid from the definitions, sweeps instead of
// rank/select, and finds neighbours through a hash map from coordinate to
// index.  Single-threaded; built with -O2 -ffp-contract=off and no fast-math so
// every fp32 operation is one IEEE round-to-nearest-even step.
//
// Sources (the pages):
//  * openvdb PR #2258 "VBM select-based inverse-map decode", "A/B": the 7-point
//    Laplacian, the 27-tap box and a 19-tap WENO consumer as the downstream
//    stencil consumers; the 19-tap shape is the centre plus three voxels each
//    way along every axis (the reach of a fifth-order WENO stencil).
//  * openvdb PR #2262 "NanoVDB VBM: Streaming box-stencil", section "What
//    changed": in an index grid a stencil resolves to indices, index 0 means
//    "no active voxel" and is skipped, a filter gathers sidecar[index*C + ch]
//    and accumulates per channel, taps are visited in the order
//    t = (di+1)*9 + (dj+1)*3 + (dk+1).
//  * openvdb PR #2258 "VBM select-based inverse-map decode", sections
//    "Summary" and "What changed": a block of BlockWidth slots; each slot's
//    leaf is the block's first leaf plus the number of leaf starts (jumpMap
//    bits) at or before it; the voxel is found through the leaf's 512-bit
//    value mask and its 9-bit prefix-sum directory; the old decode swept all
//    512 voxel slots of every leaf.  "Validation": final partial blocks and
//    beyond-last-active sentinels.
//  * openvdb PR #2263 "Alternative stencil resolvers for VoxelBlockManager",
//    "Summary" (27-tap box and 7-tap cross shapes) and "Built on the
//    register-decode API" (spanned leaves = 1 + popcount(jumpMap)).
//
// Readings where the pages leave a step open (each is listed in the design
// notes of the repository):
//  * leaves are 8^3 cells keyed by floor(p/8); voxel offset in a leaf is
//    x-major: o = (x mod 8)*64 + (y mod 8)*8 + (z mod 8);
//  * active indices are 1..N, assigned in tree order: root tile
//    floor(p/4096) lexicographic (signed), then the 32^3 upper-node slot
//    floor((p mod 4096)/128) x-major, then the 16^3 lower-node slot
//    floor((p mod 128)/8) x-major, then the voxel offset o;
//  * leafFirst of a leaf = index of its first active voxel;
//  * prefix directory: one 64-bit word holding 7 fields of 9 bits, field k
//    (bits 9k..9k+8) = number of active voxels in mask words 0..k;
//  * block b covers indices 1+b*W .. min(N, (b+1)*W); firstLeafID = leaf of
//    index 1+b*W; jumpMap bit s set iff slot s >= 1 holds an index that starts
//    a new leaf;
//  * decode sentinels: leafIndex 0xFFFFFFFF, voxelOffset 0xFFFF;
//  * di runs along x, dj along y, dk along z;
//  * cross taps: the box taps with |di|+|dj|+|dk| <= 1 in ascending box order;
//  * 19-tap axis stencil: the offsets with at most one nonzero component of
//    magnitude <= 3, in ascending lexicographic (di, dj, dk) order (centre = 9);
//    its consumer accumulates the 19 taps like the box and cross consumers;
//  * box filter = plain sum (no division); cross sum = sum over 7 taps;
//    7-point Laplacian = (sum of the active face taps, in cross order) minus
//    the separately rounded product 6*centre;
//  * WENO consumer on the 19 axis taps (the pages name it, without its
//    arithmetic): per channel the squared norm of the Godunov upwind gradient
//    built from fifth-order WENO one-sided derivatives (Jiang and Shu,
//    "Efficient implementation of weighted ENO schemes", J. Comput. Phys. 126,
//    1996; the Hamilton-Jacobi form of Jiang and Peng, SIAM J. Sci. Comput. 21,
//    2000), unit voxel spacing, epsilon 1e-6.  An inactive tap takes the value
//    of sidecar row 0 (index 0, the background).  The fp32 evaluation order is
//    fixed operation by operation in weno5() and weno_norm_sq() below.

#include <algorithm>
#include <array>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

namespace {

int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
  return q;
}
int64_t floor_mod(int64_t a, int64_t b) { return a - b * floor_div(a, b); }

struct Coord {
  int64_t x, y, z;
};

// The 12 components that order active voxels: root tile, upper-node slot,
// lower-node slot, voxel-in-leaf position; compared lexicographically.
std::array<int64_t, 12> tree_order_key(const Coord& p) {
  return {floor_div(p.x, 4096),        floor_div(p.y, 4096),        floor_div(p.z, 4096),
          floor_mod(p.x, 4096) / 128,  floor_mod(p.y, 4096) / 128,  floor_mod(p.z, 4096) / 128,
          floor_mod(p.x, 128) / 8,     floor_mod(p.y, 128) / 8,     floor_mod(p.z, 128) / 8,
          floor_mod(p.x, 8),           floor_mod(p.y, 8),           floor_mod(p.z, 8)};
}

int voxel_offset_in_leaf(const Coord& p) {
  return int(floor_mod(p.x, 8) * 64 + floor_mod(p.y, 8) * 8 + floor_mod(p.z, 8));
}

Coord leaf_origin_of(const Coord& p) {
  return {8 * floor_div(p.x, 8), 8 * floor_div(p.y, 8), 8 * floor_div(p.z, 8)};
}

// coordinates are limited to |c| < 2^20, so three biased 21-bit fields pack a key
uint64_t pack(const Coord& p) {
  const int64_t bias = int64_t(1) << 20;
  return (uint64_t(p.x + bias) << 42) | (uint64_t(p.y + bias) << 21) | uint64_t(p.z + bias);
}

struct Grid {
  std::vector<Coord> voxel;                       // voxel[g-1] = coordinate of index g
  std::unordered_map<uint64_t, uint64_t> index;   // coordinate -> index (absent = inactive)
  std::vector<uint32_t> leaf_of;                  // leaf_of[g] for g = 1..N (entry 0 unused)
  std::vector<Coord> leaf_origin;                 // per leaf, in leaf order
  std::vector<uint64_t> leaf_first;               // per leaf: index of its first active voxel
};

// The 27 box offsets in tap order t = (di+1)*9 + (dj+1)*3 + (dk+1).
Coord box_offset(int t) { return {t / 9 - 1, (t / 3) % 3 - 1, t % 3 - 1}; }

// The cross: box taps with |di|+|dj|+|dk| <= 1, ascending.
std::vector<int> cross_taps() {
  std::vector<int> taps;
  for (int t = 0; t < 27; ++t) {
    Coord d = box_offset(t);
    if (std::abs(d.x) + std::abs(d.y) + std::abs(d.z) <= 1) taps.push_back(t);
  }
  return taps;
}

// The 19 axis offsets: at most one nonzero component, of magnitude <= 3, in
// ascending lexicographic (di, dj, dk) order.
std::vector<Coord> axis19_offsets() {
  std::vector<Coord> v;
  for (int di = -3; di <= 3; ++di)
    for (int dj = -3; dj <= 3; ++dj)
      for (int dk = -3; dk <= 3; ++dk)
        if ((di != 0) + (dj != 0) + (dk != 0) <= 1) v.push_back({di, dj, dk});
  return v;
}

// Fifth-order WENO one-sided derivative from five consecutive differences
// a..e of the field along one axis, ordered away from the upwind side (for the
// left-biased derivative a = u[-2]-u[-3], ..., e = u[2]-u[1]).  Three
// third-order candidates, their smoothness indicators, and the nonlinear
// weights built from the ideal weights 1/10, 6/10, 3/10 (scaled by 10, which
// the normalisation removes) as in Jiang and Shu (1996), section 2.  Every
// operation is one fp32 rounding in the order written.
float weno5(float a, float b, float c, float d, float e) {
  const float eps = 1.0e-6f;
  // candidate derivatives on the three sub-stencils
  const float p1 = ((2.0f * a - 7.0f * b) + 11.0f * c) / 6.0f;
  const float p2 = ((-b + 5.0f * c) + 2.0f * d) / 6.0f;
  const float p3 = ((2.0f * c + 5.0f * d) - e) / 6.0f;
  // smoothness indicators: 13/12 (second difference)^2 + 1/4 (first-order term)^2
  const float q1 = (a - 2.0f * b) + c, r1 = (a - 4.0f * b) + 3.0f * c;
  const float q2 = (b - 2.0f * c) + d, r2 = b - d;
  const float q3 = (c - 2.0f * d) + e, r3 = (3.0f * c - 4.0f * d) + e;
  const float s1 = (13.0f * (q1 * q1)) / 12.0f + (r1 * r1) * 0.25f;
  const float s2 = (13.0f * (q2 * q2)) / 12.0f + (r2 * r2) * 0.25f;
  const float s3 = (13.0f * (q3 * q3)) / 12.0f + (r3 * r3) * 0.25f;
  const float t1 = s1 + eps, t2 = s2 + eps, t3 = s3 + eps;
  const float w1 = 1.0f / (t1 * t1), w2 = 6.0f / (t2 * t2), w3 = 3.0f / (t3 * t3);
  return ((w1 * p1 + w2 * p2) + w3 * p3) / ((w1 + w2) + w3);
}

// Godunov's upwind choice for |grad u|^2 along one axis from the left- and
// right-biased derivatives dm, dp; `outside` (centre value > 0) selects the
// branch for motion along +grad u, otherwise along -grad u.
float godunov_sq(float dm, float dp, bool outside) {
  const float lo = outside ? (dm > 0.0f ? dm : 0.0f) : (dm < 0.0f ? dm : 0.0f);
  const float hi = outside ? (dp < 0.0f ? dp : 0.0f) : (dp > 0.0f ? dp : 0.0f);
  const float a = lo * lo, b = hi * hi;
  return a > b ? a : b;
}

uint64_t lookup(const Grid& g, const Coord& q) {
  auto it = g.index.find(pack(q));
  return it == g.index.end() ? 0 : it->second;
}

uint64_t offset_index(const Grid& g, uint64_t idx, const Coord& d) {
  const Coord& p = g.voxel[idx - 1];
  return lookup(g, Coord{p.x + d.x, p.y + d.y, p.z + d.z});
}

uint64_t tap_index(const Grid& g, uint64_t idx, int t) { return offset_index(g, idx, box_offset(t)); }

int64_t n_blocks(int64_t n_active, int log2w) {
  int64_t w = int64_t(1) << log2w;
  return (n_active + w - 1) / w;
}

}  // namespace

extern "C" {

// Builds the oracle's index grid from n coordinates (int32 x,y,z triples, any
// order, duplicates allowed).  Returns NULL for a coordinate with |c| >= 2^20 - 1
// (so that every neighbour coordinate still packs into three 21-bit fields).
void* oracle_create(const int32_t* ijk, int64_t n) {
  std::vector<Coord> pts;
  pts.reserve(size_t(n));
  for (int64_t i = 0; i < n; ++i) {
    Coord p{ijk[3 * i], ijk[3 * i + 1], ijk[3 * i + 2]};
    const int64_t lim = (int64_t(1) << 20) - 1;
    if (p.x <= -lim || p.x >= lim || p.y <= -lim || p.y >= lim || p.z <= -lim || p.z >= lim) return nullptr;
    pts.push_back(p);
  }
  std::vector<std::pair<std::array<int64_t, 12>, Coord>> keyed;
  keyed.reserve(pts.size());
  for (const Coord& p : pts) keyed.push_back({tree_order_key(p), p});
  std::sort(keyed.begin(), keyed.end(),
            [](const auto& a, const auto& b) { return a.first < b.first; });
  keyed.erase(std::unique(keyed.begin(), keyed.end(),
                          [](const auto& a, const auto& b) { return a.first == b.first; }),
              keyed.end());

  Grid* g = new (std::nothrow) Grid();
  if (!g) return nullptr;
  g->voxel.reserve(keyed.size());
  g->leaf_of.assign(keyed.size() + 1, 0);
  for (size_t i = 0; i < keyed.size(); ++i) {
    const Coord& p = keyed[i].second;
    uint64_t idx = uint64_t(i) + 1;
    g->voxel.push_back(p);
    g->index[pack(p)] = idx;
    Coord o = leaf_origin_of(p);
    bool new_leaf = g->leaf_origin.empty() || g->leaf_origin.back().x != o.x ||
                    g->leaf_origin.back().y != o.y || g->leaf_origin.back().z != o.z;
    if (new_leaf) {
      g->leaf_origin.push_back(o);
      g->leaf_first.push_back(idx);
    }
    g->leaf_of[idx] = uint32_t(g->leaf_origin.size() - 1);
  }
  return g;
}

void oracle_destroy(void* h) { delete static_cast<Grid*>(h); }

int64_t oracle_n_active(const void* h) { return int64_t(static_cast<const Grid*>(h)->voxel.size()); }
int64_t oracle_n_leaves(const void* h) { return int64_t(static_cast<const Grid*>(h)->leaf_origin.size()); }
int64_t oracle_n_blocks(const void* h, int log2w) { return n_blocks(oracle_n_active(h), log2w); }

// coords[(g-1)*3 + c] = coordinate c of index g, g = 1..N
void oracle_voxels(const void* h, int32_t* coords) {
  const Grid& g = *static_cast<const Grid*>(h);
  for (size_t i = 0; i < g.voxel.size(); ++i) {
    coords[3 * i] = int32_t(g.voxel[i].x);
    coords[3 * i + 1] = int32_t(g.voxel[i].y);
    coords[3 * i + 2] = int32_t(g.voxel[i].z);
  }
}

// Per leaf l (in leaf order): origin[3l..3l+2], mask[8l..8l+7] (bit o of the
// 512-bit value mask is bit o%64 of word o/64), first[l], prefix[l].
void oracle_leaves(const void* h, int32_t* origin, uint64_t* mask, uint64_t* first, uint64_t* prefix) {
  const Grid& g = *static_cast<const Grid*>(h);
  const size_t L = g.leaf_origin.size();
  std::vector<uint64_t> m(L * 8, 0);
  for (size_t i = 0; i < g.voxel.size(); ++i) {
    uint32_t l = g.leaf_of[i + 1];
    int o = voxel_offset_in_leaf(g.voxel[i]);
    m[l * 8 + size_t(o / 64)] |= uint64_t(1) << (o % 64);
  }
  for (size_t l = 0; l < L; ++l) {
    origin[3 * l] = int32_t(g.leaf_origin[l].x);
    origin[3 * l + 1] = int32_t(g.leaf_origin[l].y);
    origin[3 * l + 2] = int32_t(g.leaf_origin[l].z);
    first[l] = g.leaf_first[l];
    uint64_t dir = 0, count = 0;
    for (int w = 0; w < 8; ++w) {
      mask[l * 8 + w] = m[l * 8 + w];
      for (int b = 0; b < 64; ++b)
        if ((m[l * 8 + w] >> b) & 1) ++count;
      if (w < 7) dir |= count << (9 * w);
    }
    prefix[l] = dir;
  }
}

// VBM block metadata for BlockWidth W = 2^log2w: first_leaf[b], and the W-bit
// jumpMap of block b in words jump[b*(W/64) .. b*(W/64) + W/64 - 1].
void oracle_blocks(const void* h, int log2w, uint32_t* first_leaf, uint64_t* jump) {
  const Grid& g = *static_cast<const Grid*>(h);
  const int64_t N = int64_t(g.voxel.size());
  const int64_t W = int64_t(1) << log2w;
  const int64_t words = W / 64;
  const int64_t nb = n_blocks(N, log2w);
  for (int64_t b = 0; b < nb; ++b) {
    first_leaf[b] = g.leaf_of[size_t(1 + b * W)];
    for (int64_t k = 0; k < words; ++k) jump[b * words + k] = 0;
    for (int64_t s = 1; s < W; ++s) {
      int64_t idx = 1 + b * W + s;
      if (idx <= N && g.leaf_of[size_t(idx)] != g.leaf_of[size_t(idx - 1)])
        jump[b * words + s / 64] |= uint64_t(1) << (s % 64);
    }
  }
}

// Inverse maps by a sequential sweep over every leaf's 512 voxel positions:
// slot (g-1) receives (leaf, offset) of index g; slots beyond N of the last
// block receive the sentinels.  Arrays hold n_blocks*W entries.
void oracle_decode(const void* h, int log2w, uint32_t* leaf_index, uint16_t* voxel_offset) {
  const Grid& g = *static_cast<const Grid*>(h);
  const size_t L = g.leaf_origin.size();
  std::vector<uint64_t> m(L * 8, 0);
  for (size_t i = 0; i < g.voxel.size(); ++i) {
    int o = voxel_offset_in_leaf(g.voxel[i]);
    m[g.leaf_of[i + 1] * 8 + size_t(o / 64)] |= uint64_t(1) << (o % 64);
  }
  int64_t slot = 0;
  for (size_t l = 0; l < L; ++l)
    for (int o = 0; o < 512; ++o)
      if ((m[l * 8 + size_t(o / 64)] >> (o % 64)) & 1) {
        leaf_index[slot] = uint32_t(l);
        voxel_offset[slot] = uint16_t(o);
        ++slot;
      }
  const int64_t total = n_blocks(int64_t(g.voxel.size()), log2w) << log2w;
  for (; slot < total; ++slot) {
    leaf_index[slot] = 0xFFFFFFFFu;
    voxel_offset[slot] = 0xFFFF;
  }
}

// Raw stencil taps for the m indices in idx[]: taps[i*shape + j] = index of
// tap j of voxel idx[i] (0 = inactive).  shape 27 = box, 7 = cross, 19 = axis.
int oracle_taps_rows(const void* h, int shape, const uint64_t* idx, int64_t m, uint64_t* taps) {
  const Grid& g = *static_cast<const Grid*>(h);
  std::vector<Coord> offsets;
  if (shape == 27) {
    for (int t = 0; t < 27; ++t) offsets.push_back(box_offset(t));
  } else if (shape == 7) {
    for (int t : cross_taps()) offsets.push_back(box_offset(t));
  } else if (shape == 19) {
    offsets = axis19_offsets();
  } else {
    return -1;
  }
  for (int64_t i = 0; i < m; ++i)
    for (int j = 0; j < shape; ++j) taps[i * shape + j] = offset_index(g, idx[i], offsets[size_t(j)]);
  return 0;
}

// 19-tap axis filter for the m indices in idx[]: out[i*C + ch] = fp32 sum, in
// tap order, of sidecar[tap*C + ch] over the active taps of voxel idx[i].
void oracle_axis_rows(const void* h, const float* sidecar, int C, const uint64_t* idx, int64_t m, float* out) {
  const Grid& g = *static_cast<const Grid*>(h);
  const std::vector<Coord> offsets = axis19_offsets();
  for (int64_t i = 0; i < m; ++i) {
    uint64_t tap[19];
    for (int j = 0; j < 19; ++j) tap[j] = offset_index(g, idx[i], offsets[size_t(j)]);
    for (int ch = 0; ch < C; ++ch) {
      float acc = 0.0f;
      for (int j = 0; j < 19; ++j)
        if (tap[j]) acc += sidecar[tap[j] * uint64_t(C) + uint64_t(ch)];
      out[i * C + ch] = acc;
    }
  }
}

// WENO consumer for the m indices in idx[]: out[i*C + ch] = squared norm of
// the Godunov upwind gradient of channel ch at voxel idx[i].  Per axis the
// seven values u[-3..3] come from the voxel's axis taps (an inactive tap reads
// sidecar row 0); the six differences d[k] = u[k] - u[k-1], k = -2..3, give
// the left-biased derivative weno5(d[-2], d[-1], d[0], d[1], d[2]) and the
// right-biased one weno5(d[3], d[2], d[1], d[0], d[-1]); the axes are summed
// x, then y, then z.
void oracle_weno_rows(const void* h, const float* sidecar, int C, const uint64_t* idx, int64_t m, float* out) {
  const Grid& g = *static_cast<const Grid*>(h);
  for (int64_t i = 0; i < m; ++i) {
    const Coord& p = g.voxel[idx[i] - 1];
    uint64_t tap[3][7];  // [axis][k + 3]
    for (int axis = 0; axis < 3; ++axis)
      for (int k = -3; k <= 3; ++k) {
        Coord q = p;
        if (axis == 0) q.x += k;
        if (axis == 1) q.y += k;
        if (axis == 2) q.z += k;
        tap[axis][k + 3] = lookup(g, q);
      }
    for (int ch = 0; ch < C; ++ch) {
      const float centre = sidecar[idx[i] * uint64_t(C) + uint64_t(ch)];
      const bool outside = centre > 0.0f;
      float sum = 0.0f;
      for (int axis = 0; axis < 3; ++axis) {
        float u[7];
        for (int k = 0; k < 7; ++k) u[k] = sidecar[tap[axis][k] * uint64_t(C) + uint64_t(ch)];  // index 0: row 0
        float d[6];  // d[j] = u[j+1] - u[j], i.e. the differences k = -2..3
        for (int j = 0; j < 6; ++j) d[j] = u[j + 1] - u[j];
        const float dm = weno5(d[0], d[1], d[2], d[3], d[4]);
        const float dp = weno5(d[5], d[4], d[3], d[2], d[1]);
        const float gsq = godunov_sq(dm, dp, outside);
        sum = axis == 0 ? gsq : sum + gsq;
      }
      out[i * C + ch] = sum;
    }
  }
}

// Box filter for the m indices in idx[]: out[i*C + ch] = fp32 sum, in tap
// order, of sidecar[tap*C + ch] over the active taps of voxel idx[i].
void oracle_box_rows(const void* h, const float* sidecar, int C, const uint64_t* idx, int64_t m, float* out) {
  const Grid& g = *static_cast<const Grid*>(h);
  for (int64_t i = 0; i < m; ++i) {
    uint64_t tap[27];
    for (int t = 0; t < 27; ++t) tap[t] = tap_index(g, idx[i], t);
    for (int ch = 0; ch < C; ++ch) {
      float acc = 0.0f;
      for (int t = 0; t < 27; ++t)
        if (tap[t]) acc += sidecar[tap[t] * uint64_t(C) + uint64_t(ch)];
      out[i * C + ch] = acc;
    }
  }
}

// Cross filter for the m indices in idx[]; op 0 = sum of the 7 taps,
// op 1 = 7-point Laplacian (sum of active faces) - fl(6 * centre).
int oracle_cross_rows(const void* h, const float* sidecar, int C, int op, const uint64_t* idx, int64_t m,
                      float* out) {
  const Grid& g = *static_cast<const Grid*>(h);
  if (op != 0 && op != 1) return -1;
  const std::vector<int> order = cross_taps();
  for (int64_t i = 0; i < m; ++i) {
    uint64_t tap[7];
    for (int j = 0; j < 7; ++j) tap[j] = tap_index(g, idx[i], order[size_t(j)]);
    for (int ch = 0; ch < C; ++ch) {
      float acc = 0.0f;
      for (int j = 0; j < 7; ++j) {
        if (op == 1 && order[size_t(j)] == 13) continue;  // the centre enters only as -6*centre
        if (tap[j]) acc += sidecar[tap[j] * uint64_t(C) + uint64_t(ch)];
      }
      if (op == 1) {
        float six_centre = 6.0f * sidecar[idx[i] * uint64_t(C) + uint64_t(ch)];
        acc = acc - six_centre;
      }
      out[i * C + ch] = acc;
    }
  }
  return 0;
}

// Whole-grid filters: out has (N+1)*C floats; row 0 (index 0) is written as 0.
void oracle_box_filter(const void* h, const float* sidecar, int C, float* out) {
  const int64_t N = oracle_n_active(h);
  for (int ch = 0; ch < C; ++ch) out[ch] = 0.0f;
  std::vector<uint64_t> idx(static_cast<size_t>(N));
  for (int64_t i = 0; i < N; ++i) idx[size_t(i)] = uint64_t(i) + 1;
  oracle_box_rows(h, sidecar, C, idx.data(), N, out + C);
}

int oracle_cross_filter(const void* h, const float* sidecar, int C, int op, float* out) {
  const int64_t N = oracle_n_active(h);
  for (int ch = 0; ch < C; ++ch) out[ch] = 0.0f;
  std::vector<uint64_t> idx(static_cast<size_t>(N));
  for (int64_t i = 0; i < N; ++i) idx[size_t(i)] = uint64_t(i) + 1;
  return oracle_cross_rows(h, sidecar, C, op, idx.data(), N, out + C);
}

void oracle_weno_filter(const void* h, const float* sidecar, int C, float* out) {
  const int64_t N = oracle_n_active(h);
  for (int ch = 0; ch < C; ++ch) out[ch] = 0.0f;
  std::vector<uint64_t> idx(static_cast<size_t>(N));
  for (int64_t i = 0; i < N; ++i) idx[size_t(i)] = uint64_t(i) + 1;
  oracle_weno_rows(h, sidecar, C, idx.data(), N, out + C);
}

// One weno5() evaluation (for the tests that pin it on closed forms).
float oracle_weno5(float a, float b, float c, float d, float e) { return weno5(a, b, c, d, e); }

void oracle_axis_filter(const void* h, const float* sidecar, int C, float* out) {
  const int64_t N = oracle_n_active(h);
  for (int ch = 0; ch < C; ++ch) out[ch] = 0.0f;
  std::vector<uint64_t> idx(static_cast<size_t>(N));
  for (int64_t i = 0; i < N; ++i) idx[size_t(i)] = uint64_t(i) + 1;
  oracle_axis_rows(h, sidecar, C, idx.data(), N, out + C);
}

}  // extern "C"
