// Stage 1 of the triangle multiplicative update on gfx950: LayerNorm_in, the
// gated dual projection for a and b, the pair mask, and channel-major stores.
//
// Page "Triangle Multiplicative Update (SM100 / SM103 / SM107)", section
// "Mathematics and numerics": z_in = LayerNorm(x), a = sigmoid(z g_a^T + g_a_b)
// * (z p_a^T + p_a_b) * m, b likewise; z_in rounded once to bf16 as the MMA
// operand, a and b rounded once after the fp32 mask multiply (+0.0 for m = 0).
// Section "Overview": a and b leave this stage as channel-major planes.
//
// Work decomposition. A tile is 64 pairs that share one plane row: for the
// outgoing direction the pairs (b, i, k0..k0+63), for the incoming direction
// the pairs (b, k0..k0+63, i) -- the plane row is b*N + i and the tile's 64
// pairs are 64 consecutive plane columns in both cases, so every plane store
// is a full 128-byte line per channel. A persistent block of 8 waves owns a
// channel group of 128 a-channels and 128 b-channels; each wave keeps its 32
// channels' value and gate weight rows (2 x 32 x c_z bf16) in registers for
// the whole kernel, so the weights are read once per block, not per tile.
//
// Per tile: x (64 pairs x c_z) -> registers (prefetched one tile ahead) ->
// LayerNorm (8 lanes per pair) -> z in LDS -> MFMA 32x32x16 (M = pairs,
// N = channels, K = c_z) with value and gate accumulators side by side ->
// sigmoid * value * mask in fp32 -> bf16 -> LDS transpose to [channel][pair]
// -> 16-byte coalesced plane stores.

#include "trimul_device.hpp"
#include "trimul_kernels.hpp"

namespace trimul {

namespace {

constexpr int K1_THREADS = 512;
constexpr int K1_TP = 64;          // pairs per tile
constexpr int K1_GROUP = 128;      // channels of a (and of b) per block

template <int CZ>
struct K1Smem {
  static constexpr int ZP = CZ + 8;        // z row pitch (bf16 elements)
  static constexpr int OP = K1_TP + 8;     // staging row pitch
  uint16_t z[K1_TP * ZP];
  uint16_t o[2 * K1_GROUP * OP];
  float m[K1_TP];
};

template <int CZ>
__global__ __launch_bounds__(K1_THREADS) void k1_ln_proj(const K1Args p) {
  constexpr int NV = CZ / 64;      // 16-byte chunks of a pair row per lane
  constexpr int KS = CZ / 16;      // MFMA k-steps
  using S = K1Smem<CZ>;
  __shared__ __attribute__((aligned(16))) S sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  const int group = blockIdx.y;

  // ---- per-wave weights: 32 channels of plane (wave / 4), value and gate ----
  const int plane = wave >> 2;
  const int chs = 32 * (wave & 3);                       // within the group
  const int ch = group * K1_GROUP + chs + l32;           // global channel of this lane
  const int wrow = plane * p.c + ch;                     // row of p_in / g_in
  bf16x8 wv[KS], wg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    wv[ks] = ld_frag(p.p_in + size_t(wrow) * CZ + 16 * ks + 8 * lhi);
    wg[ks] = ld_frag(p.g_in + size_t(wrow) * CZ + 16 * ks + 8 * lhi);
  }
  const float bias_v = p.p_in_b ? bf16_to_f32(p.p_in_b[wrow]) : 0.0f;
  const float bias_g = p.g_in_b ? bf16_to_f32(p.g_in_b[wrow]) : 0.0f;

  // ---- LayerNorm lane mapping: pair `lp`, sub-lane `sub` ----
  const int lp = tid >> 3;
  const int sub = tid & 7;
  u32x4 lnw[NV], lnb[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    lnw[v] = ld16(p.ln_w + 8 * sub + 64 * v);
    lnb[v] = ld16(p.ln_b + 8 * sub + 64 * v);
  }

  const int N = p.N;
  const int stride = gridDim.x;
  const size_t plane_elems = size_t(p.c) * p.B * N * p.n_pad;
  const size_t ch_stride = size_t(p.B) * N * p.n_pad;

  // x / mask element offset of the pair in slot `slot` of tile `t`.
  auto pair_index = [&](int t, int slot, int& row, int& inner) -> int {
    row = t / p.nchunk;
    inner = (t - row * p.nchunk) * K1_TP + slot;
    const int bb = row / N;
    const int fixed = row - bb * N;
    // outgoing: pair (b, fixed, inner); incoming: pair (b, inner, fixed)
    return p.incoming ? (bb * N + inner) * N + fixed : row * N + inner;
  };

  u32x4 xr[NV];
  float mr = 0.0f;
  auto prefetch = [&](int t) {
    int row, inner;
    const int pi = pair_index(t, lp, row, inner);
    if (inner < N) {
#pragma unroll
      for (int v = 0; v < NV; ++v) xr[v] = ld16(p.x + size_t(pi) * CZ + 8 * sub + 64 * v);
      mr = p.mask ? bf16_to_f32(p.mask[pi]) : 1.0f;
    } else {
#pragma unroll
      for (int v = 0; v < NV; ++v) xr[v] = u32x4{0, 0, 0, 0};
      mr = 0.0f;
    }
  };

  int t = blockIdx.x;
  if (t < p.ntiles) prefetch(t);
  for (; t < p.ntiles; t += stride) {
    int row, inner0;
    pair_index(t, 0, row, inner0);

    // ---- LayerNorm_in -> z (bf16) in LDS ----
    {
      u32x4 z[NV];
      if (inner0 + lp < N) {
        layer_norm_row<NV>(xr, lnw, lnb, p.eps, z);
      } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) z[v] = u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) st16(&sm.z[lp * S::ZP + 8 * sub + 64 * v], z[v]);
      if (sub == 0) sm.m[lp] = mr;
    }
    __syncthreads();

    // ---- prefetch the next tile while the matrix cores work ----
    if (t + stride < p.ntiles) prefetch(t + stride);

    // ---- projections: D[pair][channel] for value and gate ----
    f32x16 acc_v[2], acc_g[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc_v[mb][r] = bias_v;
        acc_g[mb][r] = bias_g;
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 a = ld_frag(&sm.z[(32 * mb + l32) * S::ZP + 16 * ks + 8 * lhi]);
        acc_v[mb] = mfma32x32x16(a, wv[ks], acc_v[mb]);
        acc_g[mb] = mfma32x32x16(a, wg[ks], acc_g[mb]);
      }
    }

    // ---- gate * value * mask, bf16, staged channel-major in LDS ----
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int m0 = 32 * mb + 8 * rg + 4 * lhi;   // first of 4 consecutive pairs
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 4 * rg + q;
          o[q] = sigmoid_f(acc_g[mb][r]) * acc_v[mb][r] * sm.m[m0 + q] + 0.0f;
        }
        const u32x2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(&sm.o[(plane * K1_GROUP + chs + l32) * S::OP + m0]) = packed;
      }
    }
    __syncthreads();

    // ---- coalesced plane stores: 256 rows (128 a + 128 b) x 64 pairs ----
#pragma unroll
    for (int it = 0; it < (2 * K1_GROUP * K1_TP / 8) / K1_THREADS; ++it) {
      const int id = it * K1_THREADS + tid;
      const int srow = id >> 3;              // staging row: plane * 128 + channel
      const int c16 = id & 7;
      const int col = inner0 + 8 * c16;
      if (col < p.n_pad) {
        const int pl = srow / K1_GROUP;
        const int gch = group * K1_GROUP + (srow - pl * K1_GROUP);
        uint16_t* dst = (pl ? p.plane_b : p.plane_a) + size_t(gch) * ch_stride + size_t(row) * p.n_pad + col;
        st16(dst, ld16(&sm.o[srow * S::OP + 8 * c16]));
      }
    }
  }
  (void)plane_elems;
}

}  // namespace

hipError_t launch_k1(const K1Args& a, int grid_x, hipStream_t stream) {
  const dim3 grid(grid_x, a.c / K1_GROUP);
  if (a.c_z == 128) {
    hipLaunchKernelGGL(k1_ln_proj<128>, grid, dim3(K1_THREADS), 0, stream, a);
  } else if (a.c_z == 256) {
    hipLaunchKernelGGL(k1_ln_proj<256>, grid, dim3(K1_THREADS), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int k1_tiles(int B, int N) { return B * N * ((N + K1_TP - 1) / K1_TP); }

}  // namespace trimul
