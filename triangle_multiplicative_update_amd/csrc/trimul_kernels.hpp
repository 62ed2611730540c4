// Launch interface between the C-ABI host code and the three gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trimul {

// Division of an index n < 2^31 by a divisor d >= 1 fixed for a launch, as a
// multiply-high, an add and a shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l, exact for
// every n below 2^32 whose sum fits 32 bits (mulhi(n, m) < n < 2^31 here).
// The kernels divide tile and row indices this way in scalar registers
// instead of the ~35-instruction division sequence.
struct FastDiv {
  uint32_t m;
  uint32_t l;
};

inline FastDiv make_fast_div(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  return FastDiv{uint32_t(m), l};
}

__device__ __forceinline__ int fast_div(int n, FastDiv f) {
  return int((__umulhi(uint32_t(n), f.m) + uint32_t(n)) >> f.l);
}

// Stage 1: LayerNorm_in + gated dual projection + mask -> planes a, b.
struct K1Args {
  const uint16_t* x;        // [B, N, N, c_z]
  const uint16_t* mask;     // [B, N, N] or nullptr
  const uint16_t* ln_w;     // [c_z]
  const uint16_t* ln_b;     // [c_z]
  const uint16_t* p_in;     // [2c, c_z]
  const uint16_t* p_in_b;   // [2c] or nullptr
  const uint16_t* g_in;     // [2c, c_z]
  const uint16_t* g_in_b;   // [2c] or nullptr
  uint16_t* plane_a;        // [c, B*N, n_pad]
  uint16_t* plane_b;        // [c, B*N, n_pad]
  int B, N, n_pad, c_z, c;
  int incoming;
  int nchunk;               // tiles per plane row: ceil(N / 64)
  int ntiles;               // B * N * nchunk
  FastDiv div_nchunk, div_N;
  float eps;
};

// Stage 2: per-channel contraction y(ch, r, j) = sum_k a(ch, r, k) b(ch, r', k).
constexpr int K2_TILE_256P = 0;   // 256 x 256 tiles, persistent blocks
constexpr int K2_TILE_128 = 1;    // 128 x 128 tiles, one block per tile
struct K2Args {
  const uint16_t* plane_a;
  const uint16_t* plane_b;
  uint16_t* plane_y;
  int B, N, n_pad, c;
  int tile;                 // K2_TILE_*, chosen by k2_plan
  int tiles_m, tiles_n;     // output tiles per (channel, batch) matrix
  int nblocks;              // tiles in all
};

// Stage 3: LayerNorm_out + LayerNorm_in recomputed + gated output projection.
struct K3Args {
  const uint16_t* plane_y;  // [c, B*N, n_pad]
  const uint16_t* x;        // [B, N, N, c_z]
  const uint16_t* ln_in_w;
  const uint16_t* ln_in_b;
  const uint16_t* ln_out_w;  // [c]
  const uint16_t* ln_out_b;  // [c]
  const uint16_t* p_out;    // [c_z, c]
  const uint16_t* p_out_b;  // [c_z] or nullptr
  const uint16_t* g_out;    // [c_z, c_z]
  const uint16_t* g_out_b;  // [c_z] or nullptr
  uint16_t* out;            // [B, N, N, c_z]
  int B, N, n_pad, c_z, c;
  int nchunk;
  int ntiles;
  FastDiv div_nchunk;
  float eps;
};

hipError_t launch_k1(const K1Args& a, int grid_x, hipStream_t stream);
hipError_t launch_k2(const K2Args& a, int max_blocks, hipStream_t stream);
hipError_t launch_k3(const K3Args& a, int grid_x, hipStream_t stream);

int k1_tiles(int B, int N);
int k3_tiles(int B, int N);
// the contraction's tile for the shape set in a (tile, tiles_m, tiles_n, nblocks)
void k2_plan(K2Args& a);

}  // namespace trimul
