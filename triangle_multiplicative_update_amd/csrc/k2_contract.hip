// Stage 2 of the triangle multiplicative update on gfx950: the per-channel
// contraction, one batched bf16 GEMM with fp32 accumulation.
//
// Page "Triangle Multiplicative Update (SM100 / SM103 / SM107)", section
// "Overview": y[c][i, j] = sum_k a[c][i, k] b[c][j, k] (outgoing) or
// sum_k a[c][k, i] b[c][k, j] (incoming), batch = c * B; section "Mathematics
// and numerics": y accumulated in fp32 and rounded once to bf16.
//
// Stage 1 writes the incoming planes with the pair index order swapped, so in
// both directions this kernel computes Y = A B^T on row-major [N x n_pad]
// matrices with k contiguous in both operands: the form the matrix cores read
// without a transpose. n_pad is a multiple of 64 and the padded columns hold
// +0.0, so the k loop has no tail.
//
// Tile: 256 x 256 outputs per block of 8 waves (2 x 4), each wave 128 (i) x
// 64 (j) as 4 x 2 v_mfma_f32_32x32x16_bf16 blocks. K advances 64 columns per
// step through a 2-stage LDS ring filled by direct global->LDS loads
// (global_load_lds_dwordx4), one step ahead of the matrix cores, one barrier
// per step. This runs as a persistent kernel (k2_contract_p: one block per CU
// looping over its tiles, the next tile's first fill overlapping the
// epilogue). Up to N = 128, where 256 x 256 tiles are mostly padding, the
// contraction runs on 128 x 128 tiles instead, one block each (k2_plan). The
// ring is laid out in 256-byte lines (one line of the 64 four-byte banks)
// holding 4 rows of 32 k each, with the 16-byte chunk index XOR-ed by the
// line index, so the 16 lanes of a fragment read hit 16 distinct bank
// groups. Rows past N are clamped to row N-1 (their results are discarded).
// The epilogue stages the bf16 tile in LDS and writes 512-byte row segments
// of y. Blocks are numbered so that the tiles of one (channel, batch) matrix
// run on one XCD and share its L2.

#include "trimul_device.hpp"
#include "trimul_kernels.hpp"

namespace trimul {

namespace {

constexpr int K2_THREADS = 512;

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Block tile BM (i) x BN (j), k step BK, STAGES-deep ring, 8 waves as WM x WN.
template <int BM_, int BN_, int BK_, int STAGES_, int WM_, int WN_>
struct K2Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, WM = WM_, WN = WN_;
  static_assert(WM * WN == 8, "8 waves");
  static constexpr int KC = BK / 8;              // 16-byte chunks per row per step
  static constexpr int RPL = 16 / KC;            // rows per 256-byte LDS line
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int RING_BYTES = STAGES * STAGE_BYTES;
  static constexpr int IA = A_BYTES / 1024 / 8;  // 1-KiB load instructions per wave per step
  static constexpr int IB = B_BYTES / 1024 / 8;
  static constexpr int PER_STEP = IA + IB;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / 32, NJ = WTN / 32;
  static constexpr int YP = BN * 2 + 16;         // epilogue row pitch (bytes)
  static constexpr int SMEM = (BM * YP > RING_BYTES) ? BM * YP : RING_BYTES;
  static_assert(IA * 8 * 1024 == A_BYTES && IB * 8 * 1024 == B_BYTES, "whole instructions");
  static_assert(SMEM <= 160 * 1024, "LDS");

  // Byte offset in an operand tile of the 16-byte chunk (row r, k-chunk c):
  // 256-byte lines of RPL rows, chunk index XOR-ed by the line index.
  __device__ __forceinline__ static int off(int r, int c) {
    const int line = r / RPL;
    const int q = ((r % RPL) * KC + c) ^ (line & 15);
    return (line * 16 + q) * 16;
  }
  // inverse: the (row, chunk) that lands on chunk P of a tile
  __device__ __forceinline__ static void src(int P, int& r, int& c) {
    const int line = P >> 4;
    const int x = (P & 15) ^ (line & 15);
    r = line * RPL + x / KC;
    c = x % KC;
  }
};

}  // namespace

// (kept outside the unnamed namespace: the host stubs of template kernels
// must have external linkage to be emitted for every instantiation)
template <int BM, int BN, int BK, int STAGES, int WM, int WN>
__global__ __launch_bounds__(K2_THREADS) void k2_contract(const K2Args p) {
  using C = K2Cfg<BM, BN, BK, STAGES, WM, WN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  const int wm = wave / C::WN;
  const int wn = wave % C::WN;

  int logical = blockIdx.x;
  const int nb = p.nblocks;
  if ((nb & 7) == 0) logical = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  const int per_mat = p.tiles_m * p.tiles_n;
  const int mat = logical / per_mat;          // = ch * B + b
  const int tile = logical - mat * per_mat;
  const int tm = tile / p.tiles_n;
  const int tn = tile - tm * p.tiles_n;
  const int N = p.N, ld = p.n_pad;
  const int i0 = tm * C::BM, j0 = tn * C::BN;
  const size_t base = size_t(mat) * N * ld;

  // this lane's load sources as byte offsets into the planes (every plane is
  // below 2^31 bytes); rows past N clamp to N - 1
  uint32_t srcA[C::IA], srcB[C::IB];
#pragma unroll
  for (int t = 0; t < C::IA; ++t) {
    int r, c;
    C::src((wave * C::IA + t) * 64 + lane, r, c);
    srcA[t] = uint32_t((base + size_t(min(i0 + r, N - 1)) * ld + 8 * c) * 2);
  }
#pragma unroll
  for (int t = 0; t < C::IB; ++t) {
    int r, c;
    C::src((wave * C::IB + t) * 64 + lane, r, c);
    srcB[t] = uint32_t((base + size_t(min(j0 + r, N - 1)) * ld + 8 * c) * 2);
  }
  auto issue = [&](int step) {
    uint8_t* st = smem + (step % C::STAGES) * C::STAGE_BYTES;
    const uint16_t* ga = p.plane_a + step * C::BK;
    const uint16_t* gb = p.plane_b + step * C::BK;
#pragma unroll
    for (int t = 0; t < C::IA; ++t) load_lds16_asm(ga, srcA[t], st + (wave * C::IA + t) * 1024);
#pragma unroll
    for (int t = 0; t < C::IB; ++t) load_lds16_asm(gb, srcB[t], st + C::A_BYTES + (wave * C::IB + t) * 1024);
  };

  constexpr int SUB = C::BK / 16;
  int offA[C::MI][SUB], offB[C::NJ][SUB];
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) offA[mi][s] = C::off(wm * C::WTM + 32 * mi + l32, 2 * s + lhi);
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) offB[nj][s] = C::A_BYTES + C::off(wn * C::WTN + 32 * nj + l32, 2 * s + lhi);
  }

  f32x16 acc[C::MI][C::NJ];
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;

  const int nk = ld / C::BK;
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < nk) issue(s);

  for (int kt = 0; kt < nk; ++kt) {
    // step kt's loads are done once at most those of the later issued steps remain
    const int later = min(C::STAGES - 2, nk - 1 - kt);
    if (later >= 3) wait_vm<3 * C::PER_STEP>();
    else if (later == 2) wait_vm<2 * C::PER_STEP>();
    else if (later == 1) wait_vm<C::PER_STEP>();
    else wait_vm<0>();
    // an LDS-only barrier: __syncthreads() would also drain the loads in
    // flight for the later steps
    lds_barrier();
    if (kt + C::STAGES - 1 < nk) issue(kt + C::STAGES - 1);

    const uint8_t* st = smem + (kt % C::STAGES) * C::STAGE_BYTES;
    // fragments of sub-step s + 1 are read while the MFMAs of s run
    bf16x8 af[2][C::MI], bfr[2][C::NJ];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) af[0][mi] = ld_frag(st + offA[mi][0]);
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) bfr[0][nj] = ld_frag(st + offB[nj][0]);
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      const int cur = s & 1;
      if (s + 1 < SUB) {
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi) af[cur ^ 1][mi] = ld_frag(st + offA[mi][s + 1]);
#pragma unroll
        for (int nj = 0; nj < C::NJ; ++nj) bfr[cur ^ 1][nj] = ld_frag(st + offB[nj][s + 1]);
      }
      // D[j][i]: rows from plane b, columns from plane a, so each lane ends
      // with 4 consecutive j of one i (8 contiguous bytes of a y row)
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < C::NJ; ++nj) acc[mi][nj] = mfma32x32x16(bfr[cur][nj], af[cur][mi], acc[mi][nj]);
      // the reads first, then the MFMAs
      if (s + 1 < SUB) __builtin_amdgcn_sched_group_barrier(0x100, C::MI + C::NJ, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, C::MI * C::NJ, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  lds_barrier();   // the ring is reused as the epilogue staging area

  // ---- epilogue: bf16 tile in LDS [i][j], then 16-byte row stores ----
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
    const int ii = wm * C::WTM + 32 * mi + l32;
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int jj = wn * C::WTN + 32 * nj + 8 * rg + 4 * lhi;
        const u32x2 w = {pack_bf16x2(acc[mi][nj][4 * rg], acc[mi][nj][4 * rg + 1]),
                         pack_bf16x2(acc[mi][nj][4 * rg + 2], acc[mi][nj][4 * rg + 3])};
        *reinterpret_cast<u32x2*>(smem + ii * C::YP + jj * 2) = w;
      }
    }
  }
  lds_barrier();
  uint16_t* Y = p.plane_y + base;
  const int jrem = min(C::BN, ld - j0);       // columns inside this row (n_pad bound)
  constexpr int CPR = C::BN / 8;              // 16-byte chunks per tile row
#pragma unroll 4
  for (int it = 0; it < (C::BM * CPR) / K2_THREADS; ++it) {
    const int id = it * K2_THREADS + tid;
    const int ii = id / CPR;
    const int cc = id % CPR;
    // y is not read again by this kernel: the non-temporal hint keeps it from
    // displacing operand lines other tiles still read from the L2
    if (i0 + ii < N && 8 * cc < jrem)
      __builtin_nontemporal_store(ld16(smem + ii * C::YP + cc * 16), reinterpret_cast<u32x4*>(Y + size_t(i0 + ii) * ld + j0 + 8 * cc));
  }
}

// Persistent form of the default tile (256 x 256, k 64, two stages): one
// block per CU loops over its tiles. After a tile's last k-step it sets up
// the next tile and issues that tile's first k-step into ring stage 0, then
// stages and stores y in two 128-row halves through the LDS past stage 0,
// so the next tile's first operand fill is in flight during the epilogue and
// no block is relaunched. Tiles are handed out so that the blocks of one XCD
// work on a contiguous range of (channel, batch) matrices, as in the
// non-persistent form. The y stores are buffer stores that are always
// issued (rows past N at an offset past the end of the plane, dropped by the
// hardware), so the wait for the next tile's first fill can count exactly the
// 16 stores issued after it.
using CfgP = K2Cfg<256, 256, 64, 2, 2, 4>;
constexpr int K2P_YROWS = CfgP::BM / 2;                 // staged rows per half
constexpr int K2P_STAGE_OFF = CfgP::STAGE_BYTES;        // staging starts past ring stage 0
constexpr int K2P_SMEM = K2P_STAGE_OFF + K2P_YROWS * CfgP::YP;
static_assert(K2P_SMEM <= 160 * 1024, "LDS");
static_assert(K2P_SMEM >= CfgP::RING_BYTES, "the LDS array holds both ring stages");
static_assert(CfgP::WM == 2, "one wave row per staged half");
constexpr int K2P_STORES = 2 * (K2P_YROWS * (CfgP::BN / 8)) / K2_THREADS;   // y stores per thread per tile

__global__ __launch_bounds__(K2_THREADS) void k2_contract_p(const K2Args p) {
  using C = CfgP;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[K2P_SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  const int wm = wave / C::WN;
  const int wn = wave % C::WN;
  const int N = p.N, ld = p.n_pad;
  const int per_mat = p.tiles_m * p.tiles_n;
  const int nb = p.nblocks;                             // tiles in all
  const int G = gridDim.x;

  // this block's tiles: logical tile first + k * step, k < count
  int first, step, count;
  if ((nb & 7) == 0 && (G & 7) == 0) {
    const int per_xcd = nb >> 3, blocks_xcd = G >> 3;
    const int x = blockIdx.x & 7, q = blockIdx.x >> 3;
    first = x * per_xcd + q;
    step = blocks_xcd;
    count = q < per_xcd ? (per_xcd - q + blocks_xcd - 1) / blocks_xcd : 0;
  } else {
    first = blockIdx.x;
    step = G;
    count = first < nb ? (nb - first + G - 1) / G : 0;
  }
  if (count == 0) return;

  const uint32_t plane_bytes = uint32_t(p.c) * uint32_t(p.B) * uint32_t(N) * uint32_t(ld) * 2u;
  const auto rsrc_y = __builtin_amdgcn_make_buffer_rsrc(p.plane_y, 0, plane_bytes, 0x00020000);

  uint32_t srcA[C::IA], srcB[C::IB];                    // byte offsets into the planes
  int i0 = 0, j0 = 0;
  uint32_t ybase = 0;                                   // element offset of the tile's matrix
  auto setup = [&](int logical) {
    const int mat = logical / per_mat;                  // = ch * B + b
    const int tile = logical - mat * per_mat;
    const int tm = tile / p.tiles_n;
    const int tn = tile - tm * p.tiles_n;
    i0 = tm * C::BM;
    j0 = tn * C::BN;
    const size_t base = size_t(mat) * N * ld;
    ybase = uint32_t(base);
    // (every plane is below 2^31 bytes; rows past N clamp to N - 1)
#pragma unroll
    for (int t = 0; t < C::IA; ++t) {
      int r, c;
      C::src((wave * C::IA + t) * 64 + lane, r, c);
      srcA[t] = uint32_t((base + size_t(min(i0 + r, N - 1)) * ld + 8 * c) * 2);
    }
#pragma unroll
    for (int t = 0; t < C::IB; ++t) {
      int r, c;
      C::src((wave * C::IB + t) * 64 + lane, r, c);
      srcB[t] = uint32_t((base + size_t(min(j0 + r, N - 1)) * ld + 8 * c) * 2);
    }
  };
  auto issue = [&](int kstep) {
    uint8_t* st = smem + (kstep % C::STAGES) * C::STAGE_BYTES;
    const uint16_t* ga = p.plane_a + kstep * C::BK;
    const uint16_t* gb = p.plane_b + kstep * C::BK;
#pragma unroll
    for (int t = 0; t < C::IA; ++t) load_lds16_asm(ga, srcA[t], st + (wave * C::IA + t) * 1024);
#pragma unroll
    for (int t = 0; t < C::IB; ++t) load_lds16_asm(gb, srcB[t], st + C::A_BYTES + (wave * C::IB + t) * 1024);
  };

  constexpr int SUB = C::BK / 16;
  int offA[C::MI][SUB], offB[C::NJ][SUB];
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) offA[mi][s] = C::off(wm * C::WTM + 32 * mi + l32, 2 * s + lhi);
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) offB[nj][s] = C::A_BYTES + C::off(wn * C::WTN + 32 * nj + l32, 2 * s + lhi);
  }

  const int nk = ld / C::BK;
  setup(first);
  issue(0);
  for (int k = 0; k < count; ++k) {
    f32x16 acc[C::MI][C::NJ];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;

    for (int kt = 0; kt < nk; ++kt) {
      // step kt's fill is done once only what was issued after it remains:
      // for the first step of a later tile, the previous tile's y stores
      if (kt == 0 && k > 0) wait_vm<K2P_STORES>();
      else wait_vm<0>();
      lds_barrier();
      const uint8_t* st = smem + (kt % C::STAGES) * C::STAGE_BYTES;
      // The CU's address unit takes the direct loads in issue order, ~2 K
      // clocks for a step's 64, and a wave stalls until its own are taken.
      // Waves 0-3 (one per SIMD) issue the next step's fills at the top of
      // the step; waves 4-7, the SIMDs' second waves, after their first
      // sub-step of MFMAs, instead of stalling behind waves 0-3's loads with
      // their matrix cores idle.
      const int fill_at = wave >= 4 ? 1 : 0;
      // fragments of sub-step s + 1 are read while the MFMAs of s run
      bf16x8 af[2][C::MI], bfr[2][C::NJ];
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi) af[0][mi] = ld_frag(st + offA[mi][0]);
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj) bfr[0][nj] = ld_frag(st + offB[nj][0]);
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        if (s == fill_at && kt + 1 < nk) issue(kt + 1);
        const int cur = s & 1;
        if (s + 1 < SUB) {
#pragma unroll
          for (int mi = 0; mi < C::MI; ++mi) af[cur ^ 1][mi] = ld_frag(st + offA[mi][s + 1]);
#pragma unroll
          for (int nj = 0; nj < C::NJ; ++nj) bfr[cur ^ 1][nj] = ld_frag(st + offB[nj][s + 1]);
        }
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
          for (int nj = 0; nj < C::NJ; ++nj) acc[mi][nj] = mfma32x32x16(bfr[cur][nj], af[cur][mi], acc[mi][nj]);
        // the reads first, then the MFMAs
        if (s + 1 < SUB) __builtin_amdgcn_sched_group_barrier(0x100, C::MI + C::NJ, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, C::MI * C::NJ, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_barrier();   // every wave is done with the ring

    // the next tile's first k-step goes into ring stage 0 during the epilogue
    const int ti0 = i0, tj0 = j0;
    const uint32_t tybase = ybase;
    if (k + 1 < count) {
      setup(first + (k + 1) * step);
      issue(0);
    }

    // ---- epilogue: y in two 128-row halves through the LDS past stage 0 ----
    const int jrem = min(C::BN, ld - tj0);              // columns inside this row (n_pad bound)
    constexpr int CPR = C::BN / 8;                      // 16-byte chunks per tile row
    uint8_t* stage = smem + K2P_STAGE_OFF;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (wm == h) {
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi) {
          const int ii = 32 * mi + l32;                 // row within the half
#pragma unroll
          for (int nj = 0; nj < C::NJ; ++nj) {
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const int jj = wn * C::WTN + 32 * nj + 8 * rg + 4 * lhi;
              const u32x2 w = {pack_bf16x2(acc[mi][nj][4 * rg], acc[mi][nj][4 * rg + 1]),
                               pack_bf16x2(acc[mi][nj][4 * rg + 2], acc[mi][nj][4 * rg + 3])};
              *reinterpret_cast<u32x2*>(stage + ii * C::YP + jj * 2) = w;
            }
          }
        }
      }
      lds_barrier();
#pragma unroll
      for (int it = 0; it < (K2P_YROWS * CPR) / K2_THREADS; ++it) {
        const int id = it * K2_THREADS + tid;
        const int ii = id / CPR;
        const int cc = id % CPR;
        const int row = ti0 + K2P_YROWS * h + ii;
        // y is not read again here: non-temporal; a row past N or a chunk
        // past n_pad goes past the end of the plane and is dropped
        const uint32_t off = (row < N && 8 * cc < jrem)
                                 ? (tybase + uint32_t(row) * uint32_t(ld) + uint32_t(tj0 + 8 * cc)) * 2u
                                 : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b128(ld16(stage + ii * C::YP + cc * 16), rsrc_y, off, 0, 2);
      }
      lds_barrier();   // the staging rows are rewritten by the next half / the next fills
    }
  }
}

// the small-N tile: 128 x 128, k 64, three stages, 8 waves of 64 x 32
using CfgSmall = K2Cfg<128, 128, 64, 3, 2, 4>;
template __global__ void k2_contract<128, 128, 64, 3, 2, 4>(const K2Args);

namespace {

template <class C>
void tiles_of(int N, int& tm, int& tn) {
  tm = (N + C::BM - 1) / C::BM;
  tn = (N + C::BN - 1) / C::BN;
}

}  // namespace

// The contraction's tile for one call (page "Triangle Multiplicative Update
// (SM100 / SM103 / SM107)", section "Overview": the contraction is compiled
// for a tile chosen per N from measured runs). 256 x 256 persistent tiles
// read the fewest operand bytes per flop. Up to N = 128 they are mostly
// padding (at N = 64 a quarter of each tile's rows and columns are real
// pairs), and 128 x 128 tiles are faster: measured on the MI355X (128 x 128
// against 256 x 256), 6.7 vs 9.0 us at N = 64, 8.4 vs 11.7 us at N = 128 (c =
// 128), 9.1 vs 12.0 us at N = 128, c = 256. From N = 129 on the two are level
// or the large tile is faster: 12.5 vs 12.5 us at N = 192 and 14.3 vs 14.6 us
// at N = 256 (c = 128, although the large tiles then leave half the CUs idle),
// 34.3 vs 33.2 us at N = 384, 20.3 vs 14.8 us at N = 192, c = 256.
void k2_plan(K2Args& a) {
  int tm, tn;
  tiles_of<CfgP>(a.N, tm, tn);
  if (a.n_pad <= CfgSmall::BM) {
    a.tile = K2_TILE_128;
    tiles_of<CfgSmall>(a.N, a.tiles_m, a.tiles_n);
  } else {
    a.tile = K2_TILE_256P;
    a.tiles_m = tm;
    a.tiles_n = tn;
  }
  a.nblocks = a.tiles_m * a.tiles_n * a.c * a.B;
}

hipError_t launch_k2(const K2Args& a, int max_blocks, hipStream_t stream) {
  if (a.tile == K2_TILE_128) {
    hipLaunchKernelGGL((k2_contract<CfgSmall::BM, CfgSmall::BN, CfgSmall::BK, CfgSmall::STAGES, CfgSmall::WM,
                                    CfgSmall::WN>),
                       dim3(a.nblocks), dim3(K2_THREADS), 0, stream, a);
  } else {
    // one persistent block per CU, a multiple of 8 (one share per XCD) when possible
    int grid = a.nblocks < max_blocks ? a.nblocks : max_blocks;
    if (grid > 8) grid &= ~7;
    hipLaunchKernelGGL(k2_contract_p, dim3(grid), dim3(K2_THREADS), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace trimul
