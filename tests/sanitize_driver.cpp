// Drives the host grid builder (vbm_build) and every oracle entry point over
// coordinate files, for a build with AddressSanitizer and UndefinedBehavior-
// Sanitizer (tests/test_sanitizers_cpu.py).  File format: int64 n, then n
// int32 triples.  Exit status 0 when every call returns as documented; a
// sanitizer report aborts the process.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "vbm.h"

extern "C" {
void* oracle_create(const int32_t* ijk, int64_t n);
void oracle_destroy(void* h);
int64_t oracle_n_active(const void* h);
int64_t oracle_n_leaves(const void* h);
int64_t oracle_n_blocks(const void* h, int log2w);
void oracle_voxels(const void* h, int32_t* coords);
void oracle_leaves(const void* h, int32_t* origin, uint64_t* mask, uint64_t* first, uint64_t* prefix);
void oracle_blocks(const void* h, int log2w, uint32_t* first_leaf, uint64_t* jump);
void oracle_decode(const void* h, int log2w, uint32_t* leaf_index, uint16_t* voxel_offset);
int oracle_taps_rows(const void* h, int shape, const uint64_t* idx, int64_t m, uint64_t* taps);
void oracle_box_filter(const void* h, const float* sidecar, int C, float* out);
int oracle_cross_filter(const void* h, const float* sidecar, int C, int op, float* out);
void oracle_axis_filter(const void* h, const float* sidecar, int C, float* out);
void oracle_weno_filter(const void* h, const float* sidecar, int C, float* out);
}

static int fail(const char* what, const char* file) {
  std::fprintf(stderr, "FAILED %s on %s\n", what, file);
  return 1;
}

int main(int argc, char** argv) {
  for (int a = 1; a < argc; ++a) {
    FILE* f = std::fopen(argv[a], "rb");
    if (!f) return fail("open", argv[a]);
    int64_t n = 0;
    if (std::fread(&n, 8, 1, f) != 1 || n < 0) return fail("read n", argv[a]);
    std::vector<int32_t> ijk(size_t(3 * n));
    if (n && std::fread(ijk.data(), 4, size_t(3 * n), f) != size_t(3 * n)) return fail("read coords", argv[a]);
    std::fclose(f);
    // host builder, every width; blob bytes read back in full
    for (int w = 6; w <= 9; ++w) {
      vbm_grid g;
      void* blob = nullptr;
      if (vbm_build(n ? ijk.data() : nullptr, n, w, &g, &blob) != VBM_OK) return fail("vbm_build", argv[a]);
      uint64_t sum = 0;
      for (uint64_t i = 0; i < g.blob_bytes; ++i) sum += static_cast<const uint8_t*>(blob)[i];
      std::printf("%s W=%d N=%llu leaves=%u blob=%llu sum=%llu\n", argv[a], 1 << w, (unsigned long long)g.n_active,
                  g.n_leaves, (unsigned long long)g.blob_bytes, (unsigned long long)sum);
      vbm_free_blob(blob);
    }
    // the oracle's coordinate limit is |c| < 2^20 - 1
    bool small = true;
    for (int32_t c : ijk) small &= c > -(1 << 20) + 1 && c < (1 << 20) - 1;
    if (!small) continue;
    void* h = oracle_create(ijk.data(), n);
    if (!h) return fail("oracle_create", argv[a]);
    const int64_t N = oracle_n_active(h), L = oracle_n_leaves(h);
    const size_t nN = size_t(N), nL = size_t(L);
    std::vector<int32_t> vox(3 * nN), origin(3 * nL);
    std::vector<uint64_t> mask(8 * nL), first(nL), prefix(nL);
    oracle_voxels(h, vox.data());
    oracle_leaves(h, origin.data(), mask.data(), first.data(), prefix.data());
    for (int w = 6; w <= 9; ++w) {
      const size_t nb = size_t(oracle_n_blocks(h, w)), slots = nb << w;
      std::vector<uint32_t> fl(nb), li(slots);
      std::vector<uint64_t> jump(nb * size_t((1 << w) / 64));
      std::vector<uint16_t> vo(slots);
      oracle_blocks(h, w, fl.data(), jump.data());
      oracle_decode(h, w, li.data(), vo.data());
    }
    std::vector<uint64_t> idx(nN);
    for (int64_t i = 0; i < N; ++i) idx[size_t(i)] = uint64_t(i) + 1;
    for (int shape : {27, 7, 19}) {
      std::vector<uint64_t> taps(nN * size_t(shape));
      if (oracle_taps_rows(h, shape, idx.data(), N, taps.data()) != 0) return fail("taps", argv[a]);
    }
    for (int C : {1, 3, 16}) {
      const size_t rows = (nN + 1) * size_t(C);
      std::vector<float> sc(rows), out(rows);
      for (size_t i = 0; i < sc.size(); ++i) sc[i] = float(int(i % 7) - 3) * 0.25f;
      oracle_box_filter(h, sc.data(), C, out.data());
      if (oracle_cross_filter(h, sc.data(), C, 0, out.data()) != 0) return fail("cross", argv[a]);
      if (oracle_cross_filter(h, sc.data(), C, 1, out.data()) != 0) return fail("laplacian", argv[a]);
      oracle_axis_filter(h, sc.data(), C, out.data());
      oracle_weno_filter(h, sc.data(), C, out.data());
    }
    oracle_destroy(h);
  }
  return 0;
}
