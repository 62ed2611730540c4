// Stage 2 of the triangle multiplicative update on gfx950: the per-channel
// contraction, one batched bf16 GEMM with fp32 accumulation.
//
// Page "Triangle Multiplicative Update (SM100 / SM103 / SM107)", section
// "Overview": y[c][i, j] = sum_k a[c][i, k] b[c][j, k] (outgoing) or
// sum_k a[c][k, i] b[c][k, j] (incoming), batch = c * B; section "Mathematics
// and numerics": y accumulated in fp32 and rounded once to bf16.
//
// Stage 1 writes the incoming planes with the pair index order swapped, so in
// both directions this kernel computes Y = A * B^T on [N x n_pad] row-major
// matrices (k contiguous in both operands): the NT form the matrix cores read
// without any transpose.
//
// Tile: 128 x 128 outputs per 256-thread block, 4 waves of 64 x 64, each a 2 x 2
// grid of v_mfma_f32_32x32x16_bf16. K advances 32 columns per step through a
// double-buffered LDS stage; the next step's global loads are in flight while
// the current step multiplies. Blocks are numbered so that the blocks of one
// (channel, batch) matrix run on one XCD and share its L2.

#include "trimul_device.hpp"
#include "trimul_kernels.hpp"

namespace trimul {

namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int K2_THREADS = 256;
constexpr int PITCH = BK + 8;     // LDS row pitch (bf16): 80 bytes

__global__ __launch_bounds__(K2_THREADS) void k2_contract(const K2Args p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware numbering: hardware block id b runs on XCD b % 8; give XCD x the
  // contiguous logical range [x * n / 8, (x + 1) * n / 8).
  int logical = blockIdx.x;
  const int nb = p.nblocks;
  if ((nb & 7) == 0) logical = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  const int per_mat = p.tiles_m * p.tiles_n;
  const int mat = logical / per_mat;          // = ch * B + b
  const int tile = logical - mat * per_mat;
  const int tm = tile / p.tiles_n;
  const int tn = tile - tm * p.tiles_n;
  const int N = p.N, ld = p.n_pad;
  const int i0 = tm * BM, j0 = tn * BN;
  const size_t base = size_t(mat) * N * ld;   // rows (ch, b, 0..N-1)
  const uint16_t* Ag = p.plane_a + base;
  const uint16_t* Bg = p.plane_b + base;

  // global -> register staging: 2 chunks of A and 2 of B per thread
  u32x4 ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int id = tid + h * K2_THREADS;
      const int r = id >> 2;
      const int kc = k0 + 8 * (id & 3);
      const bool kin = kc < ld;
      ra[h] = (kin && i0 + r < N) ? ld16(Ag + size_t(i0 + r) * ld + kc) : u32x4{0, 0, 0, 0};
      rb[h] = (kin && j0 + r < N) ? ld16(Bg + size_t(j0 + r) * ld + kc) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int id = tid + h * K2_THREADS;
      const int r = id >> 2;
      const int kk = 8 * (id & 3);
      st16(&As[buf][r * PITCH + kk], ra[h]);
      st16(&Bs[buf][r * PITCH + kk], rb[h]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  const int nk = (ld + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = ld_frag(&As[buf][(wm * 64 + 32 * mi + l32) * PITCH + kk + 8 * lhi]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bfr[ni] = ld_frag(&Bs[buf][(wn * 64 + 32 * ni + l32) * PITCH + kk + 8 * lhi]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32x32x16(af[mi], bfr[ni], acc[mi][ni]);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  // epilogue: D[m = i][n = j]; lane holds column j = l32, rows 8*(r/4) + 4*lhi + r%4
  uint16_t* Y = p.plane_y + base;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int j = j0 + wn * 64 + 32 * ni + l32;
      if (j < N) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int i = i0 + wm * 64 + 32 * mi + 8 * (r >> 2) + 4 * lhi + (r & 3);
          const uint32_t w = pack_bf16x2(acc[mi][ni][r], acc[mi][ni][r + 1]);
          if (i < N) Y[size_t(i) * ld + j] = uint16_t(w & 0xffffu);
          if (i + 1 < N) Y[size_t(i + 1) * ld + j] = uint16_t(w >> 16);
        }
      }
    }
  }
}

}  // namespace

void k2_tiles(int N, int& tiles_m, int& tiles_n) {
  tiles_m = (N + BM - 1) / BM;
  tiles_n = (N + BN - 1) / BN;
}

hipError_t launch_k2(const K2Args& a, hipStream_t stream) {
  hipLaunchKernelGGL(k2_contract, dim3(a.nblocks), dim3(K2_THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace trimul
