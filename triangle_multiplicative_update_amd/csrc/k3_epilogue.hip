// Stage 3 of the triangle multiplicative update on gfx950: LayerNorm_out over
// the channels of y, LayerNorm_in of x recomputed, and the gated output
// projection.
//
// Page "Triangle Multiplicative Update (SM100 / SM103 / SM107)", section
// "Mathematics and numerics": u = LayerNorm_c(y), out = sigmoid(z_in g_out^T +
// g_out_b) * (u p_out^T + p_out_b); u and z_in rounded once to bf16 as the MMA
// operands, out rounded once to bf16, not masked. Section "Overview": y arrives
// channel-major, out leaves pair-major.
//
// Work decomposition. A tile is 64 pairs (b, i, j0..j0+63): one row of each y
// plane (128 contiguous bytes per channel) and 64 contiguous pair rows of x
// and out. A persistent block of 8 waves keeps the output weights in registers:
// each wave owns 32 output channels (p_out and g_out rows) and one or both
// 32-pair halves of the tile.
//
// Per tile: y (c channels x 64 pairs) -> LDS transposed to [pair][channel];
// x -> registers -> LayerNorm_in (the stage-1 lane mapping, so z_in is
// bit-identical) -> LDS; LayerNorm_out in place on the y rows; MFMA 32x32x16 with
// D[out channel][pair] (A = weights, B = activations) for the value and the gate;
// sigmoid * value in fp32 -> bf16 -> LDS [pair][channel] -> 16-byte coalesced
// stores of out.

#include "trimul_device.hpp"
#include "trimul_kernels.hpp"

namespace trimul {

namespace {

constexpr int K3_THREADS = 512;
constexpr int K3_TP = 64;

template <int C>
struct K3Smem {
  static constexpr int P = C + 8;          // row pitch (bf16) of the pair-major tiles
  uint16_t y[K3_TP * P];                   // y, then u, [pair][channel]
  uint16_t z[K3_TP * P];                   // z_in [pair][channel]
  uint16_t o[K3_TP * P];                   // out staging [pair][channel]
};

template <int C>
__global__ __launch_bounds__(K3_THREADS) void k3_epilogue(const K3Args p) {
  constexpr int CZ = C;                    // c_z == c
  constexpr int NV = C / 64;
  constexpr int KS = C / 16;
  constexpr int NB = CZ / 32;              // 32-channel output blocks
  constexpr int JOBS = 2 * NB / 8;         // (channel block, pair half) jobs per wave
  using S = K3Smem<C>;
  __shared__ __attribute__((aligned(16))) S sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  // ---- wave job: output channel block nb, pair halves mb ----
  const int nb = (JOBS == 1) ? (wave % NB) : wave;
  const int mb_first = (JOBS == 1) ? (wave / NB) : 0;
  const int nrow = 32 * nb + l32;          // weight row (output channel) this lane feeds
  bf16x8 wp[KS], wg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    wp[ks] = ld_frag(p.p_out + size_t(nrow) * C + 16 * ks + 8 * lhi);
    wg[ks] = ld_frag(p.g_out + size_t(nrow) * CZ + 16 * ks + 8 * lhi);
  }
  // accumulator register r holds output channel 32*nb + 8*(r/4) + 4*lhi + r%4
  float bias_p[16], bias_g[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int n = 32 * nb + 8 * (r >> 2) + 4 * lhi + (r & 3);
    bias_p[r] = p.p_out_b ? bf16_to_f32(p.p_out_b[n]) : 0.0f;
    bias_g[r] = p.g_out_b ? bf16_to_f32(p.g_out_b[n]) : 0.0f;
  }

  // ---- LayerNorm lane mapping (same as stage 1) ----
  const int lp = tid >> 3;
  const int sub = tid & 7;
  u32x4 inw[NV], inb[NV], outw[NV], outb[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    inw[v] = ld16(p.ln_in_w + 8 * sub + 64 * v);
    inb[v] = ld16(p.ln_in_b + 8 * sub + 64 * v);
    outw[v] = ld16(p.ln_out_w + 8 * sub + 64 * v);
    outb[v] = ld16(p.ln_out_b + 8 * sub + 64 * v);
  }

  const int N = p.N;
  const size_t ch_stride = size_t(p.B) * N * p.n_pad;

  for (int t = blockIdx.x; t < p.ntiles; t += gridDim.x) {
    const int row = t / p.nchunk;                      // b * N + i
    const int j0 = (t - row * p.nchunk) * K3_TP;

    // ---- y rows of the tile -> LDS, transposed to [pair][channel] ----
#pragma unroll
    for (int it = 0; it < (C * K3_TP / 8) / K3_THREADS; ++it) {
      const int id = it * K3_THREADS + tid;
      const int ch = id >> 3;
      const int jc = id & 7;
      const int col = j0 + 8 * jc;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (col < p.n_pad) v = ld16(p.plane_y + size_t(ch) * ch_stride + size_t(row) * p.n_pad + col);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sm.y[(8 * jc + 2 * q) * S::P + ch] = uint16_t(v[q] & 0xffffu);
        sm.y[(8 * jc + 2 * q + 1) * S::P + ch] = uint16_t(v[q] >> 16);
      }
    }

    // ---- x -> LayerNorm_in -> z_in in LDS ----
    {
      const bool valid = j0 + lp < N;
      u32x4 xr[NV], z[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v)
        xr[v] = valid ? ld16(p.x + (size_t(row) * N + j0 + lp) * CZ + 8 * sub + 64 * v) : u32x4{0, 0, 0, 0};
      if (valid) {
        layer_norm_row<NV>(xr, inw, inb, p.eps, z);
      } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) z[v] = u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) st16(&sm.z[lp * S::P + 8 * sub + 64 * v], z[v]);
    }
    __syncthreads();

    // ---- LayerNorm_out in place on the pair rows of y ----
    {
      u32x4 yr[NV], u[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) yr[v] = ld16(&sm.y[lp * S::P + 8 * sub + 64 * v]);
      layer_norm_row<NV>(yr, outw, outb, p.eps, u);
#pragma unroll
      for (int v = 0; v < NV; ++v) st16(&sm.y[lp * S::P + 8 * sub + 64 * v], u[v]);
    }
    __syncthreads();

    // ---- output projection and gate: D[out channel][pair] ----
#pragma unroll
    for (int jb = 0; jb < JOBS; ++jb) {
      const int mb = mb_first + jb;
      f32x16 acc_p, acc_g;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc_p[r] = bias_p[r];
        acc_g[r] = bias_g[r];
      }
      const int prow = 32 * mb + l32;     // pair this lane feeds as the B operand
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 u = ld_frag(&sm.y[prow * S::P + 16 * ks + 8 * lhi]);
        const bf16x8 z = ld_frag(&sm.z[prow * S::P + 16 * ks + 8 * lhi]);
        acc_p = mfma32x32x16(wp[ks], u, acc_p);
        acc_g = mfma32x32x16(wg[ks], z, acc_g);
      }
      // lane holds pair 32*mb + l32 and 4 consecutive channels per register group
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = sigmoid_f(acc_g[4 * rg + q]) * acc_p[4 * rg + q];
        const u32x2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(&sm.o[prow * S::P + 32 * nb + 8 * rg + 4 * lhi]) = packed;
      }
    }
    __syncthreads();

    // ---- coalesced pair-major stores of out ----
#pragma unroll
    for (int it = 0; it < (K3_TP * CZ / 8) / K3_THREADS; ++it) {
      const int id = it * K3_THREADS + tid;
      const int pr = id / (CZ / 8);
      const int cc = id - pr * (CZ / 8);
      if (j0 + pr < N)
        st16(p.out + (size_t(row) * N + j0 + pr) * CZ + 8 * cc, ld16(&sm.o[pr * S::P + 8 * cc]));
    }
  }
}

}  // namespace

int k3_tiles(int B, int N) { return B * N * ((N + K3_TP - 1) / K3_TP); }

hipError_t launch_k3(const K3Args& a, int grid_x, hipStream_t stream) {
  if (a.c == 128) {
    hipLaunchKernelGGL(k3_epilogue<128>, dim3(grid_x), dim3(K3_THREADS), 0, stream, a);
  } else if (a.c == 256) {
    hipLaunchKernelGGL(k3_epilogue<256>, dim3(grid_x), dim3(K3_THREADS), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace trimul
