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
// Work decomposition. A tile is 64 pairs (b, i, j0..j0+63): one 128-byte row
// of each y plane and 64 contiguous pair rows of x and out; blocks of 8 waves
// are persistent. Two forms: at c = 128 the waves specialise (k3_epilogue_ws:
// four matrix waves, four LayerNorm waves, one of each per SIMD); at c = 256
// every wave runs every phase (k3_epilogue<256>). Both transpose y to
// pair-major LDS rows two channels per dword, run LayerNorm_in with the
// stage-1 lane mapping (so z_in is bit-identical) and LayerNorm_out, compute
// the value and gate with MFMA 32x32x16 as D[out channel][pair] (weights as
// the A operand, held in registers), and stage sigmoid * value as bf16 in LDS
// [pair][channel] for 16-byte coalesced stores. The y/u and z tiles use the
// 256-byte-row slot swizzle (lds_swz); the out staging tile has its own
// 8-byte-unit swizzle (ooff), both conflict-free for their accesses under
// gfx950's LDS bank model.

#include "trimul_device.hpp"
#include "trimul_kernels.hpp"

namespace trimul {

namespace {

constexpr int K3_THREADS = 512;
constexpr int K3_TP = 64;

template <int C>
struct K3Smem {
  static constexpr int RB = C * 2;         // row bytes (pair-major, no padding)
  uint8_t y[K3_TP * RB];                   // y, then u
  uint8_t z[K3_TP * RB];                   // x of the tile (direct loads), then z_in in place
  uint8_t o[K3_TP * RB];                   // out staging
  uint8_t ys[C * K3_TP * 2];               // y of the next tile, channel-major (direct loads)
  float inw[C], inb[C], outw[C], outb[C], bp[C], bg[C];   // LayerNorm affines, output biases
};

// byte offset of 16-byte slot `slot` of pair row `r` in a swizzled tile
template <int C>
__device__ __forceinline__ int soff(int r, int slot) {
  return r * (C * 2) + ((slot ^ lds_swz(r)) << 4);
}

// Out staging: 8-byte unit u of pair row r at unit u ^ (r % 32). The epilogue
// writes 32 rows x one unit per 8-byte instruction (32 distinct units: no
// conflict); the store pass reads 16-byte chunk c of row r from chunk
// c ^ ((r % 32) >> 1), with its two 8-byte halves swapped when r is odd.
template <int C>
__device__ __forceinline__ int ooff(int r, int unit) {
  return r * (C * 2) + ((unit ^ (r & 31)) << 3);
}

// c = 256 form. Every wave runs every phase of a tile. The 32 output
// channels' weights of a wave take 128 registers, so nothing is prefetched
// into registers: the next tile's y and x travel by direct global -> LDS
// loads while this tile is processed, y into a channel-major staging tile
// (issued once this tile's y has been transposed out of it), x into the z
// tile (issued once this tile's MFMAs have read z). Per tile:
//   wait for y(t); barrier
//   y staging -> pair-major y rows (two channels per dword); barrier
//   issue y(t+1); LayerNorm_out in place on the y rows; wait for this
//   wave's rows of x(t); LayerNorm_in in place on them (stage-1 lane
//   mapping); barrier
//   two (32-channel block, pair half) jobs per wave of the output projection
//   and gate into the out staging; barrier
//   issue x(t+1); pair-major stores of tile t
// x(t) is waited for after LayerNorm_out, so its loads (issued late in the
// previous tile, the z tile being their only home) have the transpose and
// LayerNorm_out to land behind. Every store is issued (a pair past N at an
// offset past the end of out, dropped by the hardware), so both waits count
// exactly: the previous tile's stores and the loads issued after the one
// waited for. The LayerNorm affines and output biases live in LDS as fp32.
template <int C>
__global__ __launch_bounds__(K3_THREADS) void k3_epilogue(const K3Args p) {
  static_assert(C == 256, "the c = 128 form is k3_epilogue_ws");
  constexpr int CZ = C;                    // c_z == c
  constexpr int NV = C / 64;               // LayerNorm chunks per lane
  constexpr int KS = C / 16;               // MFMA k-steps
  constexpr int NB = CZ / 32;              // 32-channel output blocks
  constexpr int JOBS = 2 * NB / 8;         // (channel block, pair half) jobs per wave
  constexpr int NY = (C / 2) * 8 / K3_THREADS;   // (channel pair, 8-pair chunk) items per thread
  constexpr int NST = (K3_TP * CZ / 8) / K3_THREADS;   // 16-byte out chunks per thread per tile
  constexpr int NLD = K3_TP * C * 2 / 1024 / 8;        // 1 KB direct loads per wave per tile and tensor
  static_assert(NLD == 4 && NST == 4, "wait counts below assume 4 loads and 4 stores per wave");
  using S = K3Smem<C>;
  __shared__ __attribute__((aligned(16))) S sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  const int N = p.N;
  const int G = gridDim.x;
  const int nk = int(blockIdx.x) < p.ntiles ? (p.ntiles - int(blockIdx.x) + G - 1) / G : 0;
  if (nk == 0) return;                      // the whole block: no barrier is left unmatched
  auto tile_at = [&](int k, int& row, int& j0) {
    const int t = int(blockIdx.x) + k * G;
    row = fast_div(t, p.div_nchunk);                     // b * N + i
    j0 = (t - row * p.nchunk) * K3_TP;
  };

  // ---- wave jobs: output channel block nb, both pair halves ----
  const int nb = wave;
  const int nrow = 32 * nb + l32;          // weight row (output channel) this lane feeds
  bf16x8 wp[KS], wg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    wp[ks] = ld_frag(p.p_out + size_t(nrow) * C + 16 * ks + 8 * lhi);
    wg[ks] = ld_frag(p.g_out + size_t(nrow) * CZ + 16 * ks + 8 * lhi);
  }

  // ---- LayerNorm lane mapping (same as stage 1): pair lp, sub-lane sub ----
  const int lp = tid >> 3;
  const int sub = tid & 7;
  stage_f32(sm.inw, p.ln_in_w, CZ);
  stage_f32(sm.inb, p.ln_in_b, CZ);
  stage_f32(sm.outw, p.ln_out_w, C);
  stage_f32(sm.outb, p.ln_out_b, C);
  stage_f32(sm.bp, p.p_out_b, CZ);
  stage_f32(sm.bg, p.g_out_b, CZ);

  const size_t ch_stride = size_t(p.B) * N * p.n_pad;
  const uint32_t xo_bytes = uint32_t(p.B) * uint32_t(N) * uint32_t(N) * uint32_t(CZ) * 2u;
  const auto rsrc_o = __builtin_amdgcn_make_buffer_rsrc(p.out, 0, xo_bytes, 0x00020000);

  // y of a tile -> channel-major staging, 128 bytes (64 pairs) per row. Row r
  // holds channel r ^ ((r >> 1) & 1), so that the even (and the odd) channels
  // one 16-lane cycle of the transpose reads fall in both halves of the banks.
  // Load q of wave w fills slots s = (w NLD + q) 64 + lane: row r = s / 8,
  // 8 pairs jc = s % 8. Rows 8 (w NLD + q) .. + 7 differ between loads only in
  // that multiple of 8, which the channel flip leaves alone, so one lane offset
  // plus a uniform 8 channels per load serves all NLD loads.
  const int yr = lane >> 3;
  const uint32_t yoff = (uint32_t(8 * wave * NLD + (yr ^ ((yr >> 1) & 1))) * uint32_t(ch_stride) +
                         8u * uint32_t(lane & 7)) * 2u;
  const uint32_t ystep = 8u * uint32_t(ch_stride) * 2u;
  auto load_y = [&](int row, int j0) {
    const char* base = reinterpret_cast<const char*>(p.plane_y + size_t(row) * p.n_pad + j0);
#pragma unroll
    for (int q = 0; q < NLD; ++q) load_lds16_asm(base + q * ystep, yoff, sm.ys + (wave * NLD + q) * 1024);
  };
  // x of a tile -> the z tile, 512 bytes per pair row, 16-byte chunk c of pair
  // lp at position c ^ (8 (lp & 1)) (conflict-free for the LayerNorm lane
  // mapping); a pair past N reads pair N - 1 (its results are not stored)
  auto load_x = [&](int row, int j0) {
    const char* base = reinterpret_cast<const char*>(p.x + (size_t(row) * N + j0) * CZ);
    const int last = N - 1 - j0;
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int s = (wave * NLD + q) * 64 + lane;
      const int pr = s >> 5, pos = s & 31;
      const int c = pos ^ ((pr & 1) << 3);
      const uint32_t off = (uint32_t(min(pr, last)) * CZ + 8u * uint32_t(c)) * 2u;
      load_lds16_asm(base, off, sm.z + (wave * NLD + q) * 1024);
    }
  };

  {
    int row, j0;
    tile_at(0, row, j0);
    load_y(row, j0);
    load_x(row, j0);
  }
  for (int k = 0; k < nk; ++k) {
    int row, j0, rown, j0n;
    tile_at(k, row, j0);
    tile_at(k + 1 < nk ? k + 1 : k, rown, j0n);      // the last tile loads itself again
    // y of this tile has landed: issued since, this tile's x loads (the
    // previous tile's, after its MFMAs) and the previous tile's stores
    if (k == 0) wait_vm<NLD>();
    else wait_vm<NLD + NST>();
    lds_barrier();

    // ---- y staging -> pair-major rows (two channels per dword) ----
    // item: channel pair cp = id / 8, pair chunk jc = id % 8
#pragma unroll
    for (int it = 0; it < NY; ++it) {
      const int id = it * K3_THREADS + tid;
      const int cp = id >> 3;
      const int jc = id & 7;
      const int flip = cp & 1;              // rows of channels 2 cp, 2 cp + 1 (see load_y)
      const u32x4 ya = ld16(sm.ys + ((2 * cp) ^ flip) * 128 + 16 * jc);
      const u32x4 yb = ld16(sm.ys + ((2 * cp + 1) ^ flip) * 128 + 16 * jc);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t even = __builtin_amdgcn_perm(yb[q], ya[q], 0x05040100u);   // pair 8jc + 2q
        const uint32_t odd = __builtin_amdgcn_perm(yb[q], ya[q], 0x07060302u);    // pair 8jc + 2q + 1
        const int r0 = 8 * jc + 2 * q;
        *reinterpret_cast<uint32_t*>(sm.y + soff<C>(r0, cp >> 2) + 4 * (cp & 3)) = even;
        *reinterpret_cast<uint32_t*>(sm.y + soff<C>(r0 + 1, cp >> 2) + 4 * (cp & 3)) = odd;
      }
    }
    lds_barrier();
    load_y(rown, j0n);

    // ---- LayerNorm_out in place on the pair rows of y ----
    {
      u32x4 yr[NV], u[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) yr[v] = ld16(sm.y + soff<C>(lp, sub + 8 * v));
      layer_norm_row_lds<NV>(yr, sm.outw, sm.outb, sub, p.eps, u);
#pragma unroll
      for (int v = 0; v < NV; ++v) st16(sm.y + soff<C>(lp, sub + 8 * v), u[v]);
    }

    // ---- LayerNorm_in in place: x rows of the z tile -> z_in ----
    // x of this tile has landed: issued since, the previous tile's stores
    // and the next tile's y loads. A wave's LayerNorm lanes read only the
    // pair rows that wave loaded (rows 8w .. 8w + 7), so no barrier is needed
    // between the wait and the reads; the 8 lanes of pair lp are in one wave
    // and read the whole row before any of them writes it.
    __builtin_amdgcn_sched_barrier(0);
    if (k == 0) wait_vm<NLD>();
    else wait_vm<NST + NLD>();
    {
      u32x4 xr[NV], z[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) xr[v] = ld16(sm.z + lp * (C * 2) + (((sub + 8 * v) ^ ((lp & 1) << 3)) << 4));
      layer_norm_row_lds<NV>(xr, sm.inw, sm.inb, sub, p.eps, z);
#pragma unroll
      for (int v = 0; v < NV; ++v) st16(sm.z + soff<C>(lp, sub + 8 * v), z[v]);
    }
    lds_barrier();

    // ---- output projection and gate: D[out channel][pair] ----
#pragma unroll
    for (int mb = 0; mb < JOBS; ++mb) {
      f32x16 acc_p, acc_g;
#pragma unroll
      for (int q = 0; q < 4; ++q) {   // 4 consecutive output channels per register group
        const int n = 32 * nb + 8 * q + 4 * lhi;
        const f32x4 bp4 = *reinterpret_cast<const f32x4*>(&sm.bp[n]);
        const f32x4 bg4 = *reinterpret_cast<const f32x4*>(&sm.bg[n]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc_p[4 * q + e] = bp4[e];
          acc_g[4 * q + e] = bg4[e];
        }
      }
      const int prow = 32 * mb + l32;     // pair this lane feeds as the B operand
      // soff(prow, 2 ks + lhi) = fbase + 256 (ks >> 3) + 32 ((ks & 7) ^ ft):
      // two opaque per-tile values instead of one address register per k-step
      const int fs = lds_swz(prow);
      int fbase = prow * (C * 2) + ((lhi ^ (fs & 1)) << 4);
      int ft = fs >> 1;
      asm volatile("" : "+v"(fbase), "+v"(ft));
      auto faddr = [&](int ks) { return fbase + 256 * (ks >> 3) + ((((ks & 7) ^ ft)) << 5); };
      // the u and z fragments of k-step ks + 1 are read before the MFMAs of ks
      bf16x8 uf[2], zf[2];
      uf[0] = ld_frag(sm.y + faddr(0));
      zf[0] = ld_frag(sm.z + faddr(0));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < KS) {
          const int a = faddr(ks + 1);
          uf[cur ^ 1] = ld_frag(sm.y + a);
          zf[cur ^ 1] = ld_frag(sm.z + a);
        }
        acc_p = mfma32x32x16(wp[ks], uf[cur], acc_p);
        acc_g = mfma32x32x16(wg[ks], zf[cur], acc_g);
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane holds pair 32*mb + l32 and 4 consecutive channels per register group
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = sigmoid_f(acc_g[4 * rg + q]) * acc_p[4 * rg + q];
        const u32x2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(sm.o + ooff<C>(prow, 2 * (4 * nb + rg) + lhi)) = packed;
      }
    }
    lds_barrier();
    load_x(rown, j0n);

    // ---- pair-major stores of out (a pair past N goes past the end of out:
    // 0x80000000 plus a tile base below 2^31 stays below 2^32, and is dropped) ----
    const int so = __builtin_amdgcn_readfirstlane((row * N + j0) * CZ * 2);
#pragma unroll
    for (int it = 0; it < NST; ++it) {
      const int id = it * K3_THREADS + tid;
      const int pr = id / (CZ / 8);
      const int cc = id - pr * (CZ / 8);
      u32x4 v = ld16(sm.o + pr * (C * 2) + ((cc ^ ((pr & 31) >> 1)) << 4));
      if (pr & 1) v = u32x4{v[2], v[3], v[0], v[1]};
      const uint32_t off = j0 + pr < N ? uint32_t(id) * 16u : 0x80000000u;
      buffer_store16(rsrc_o, v, off + uint32_t(so));
    }
  }
  // the last tile's loads of itself: nothing may still be writing the LDS
  // when the block ends
  wait_vm<0>();
}

// ---------------------------------------------------------------------------
// c = 128: wave-specialised form. Waves 0-3 ("matrix waves") each own one
// 32-channel output block for both pair halves: the p_out and g_out MFMAs, the
// gate, the out staging and the stores; they also load y and transpose it to
// pair-major LDS rows (cheap permutes and 4-byte writes). Waves 4-7
// ("LayerNorm waves") load x and run LayerNorm_in (the stage-1 lane mapping:
// 8 lanes per pair, so z_in is bit-identical) and LayerNorm_out, 16 pairs per
// wave, writing z and u for the matrix waves. Each SIMD holds one wave of each
// kind, so the matrix cores of one overlap the vector ALU work of the other.
// Iteration k has two barriers:
//   phase 1: matrix waves run tile k's MFMAs (u/z buffer k % 2), then
//            transpose the y of tile k+1 (in registers) into the shared y
//            rows; LayerNorm waves write z of tile k+1
//   phase 2: matrix waves run both pair halves' gates, store tile k-1 and load
//            y of tile k+3; LayerNorm waves write u of tile k+1.
// The LayerNorm waves load x of tile k+3 in phase 1, right after their
// LayerNorm_in has read the register set the loads go to (two register sets:
// x has 2 iterations to land, y 1.5); phase 2 then holds the matrix waves'
// y loads and stores alone.
// Loads are issued in every iteration (clamped to the block's last tile) and
// the stores too (past the end of out where there is nothing to store):
// vector-memory operations retire in issue order and the compiler counts the
// waits per loop, merging the paths into it, so every path must issue the same
// operations, or a wait for a load would also drain the newer ones.
constexpr int K3W_PAIRS = 16;              // pairs per LayerNorm wave

struct K3WsSmem {
  static constexpr int RB = 256;           // pair row bytes (128 bf16)
  uint8_t u[2][K3_TP * RB];                // LayerNorm_out rows
  uint8_t z[2][K3_TP * RB];                // LayerNorm_in rows
  uint8_t o[2][K3_TP * RB];                // out staging
  uint8_t y[K3_TP * RB];                   // transposed y rows of the next tile
  float bp[128], bg[128];                  // output biases, fp32 (the accumulators' initial values)
};

__global__ __launch_bounds__(K3_THREADS) void k3_epilogue_ws(const K3Args p) {
  constexpr int C = 128, CZ = 128;
  constexpr int NV = C / 64;               // LayerNorm chunks per lane
  constexpr int KS = C / 16;               // MFMA k-steps
  constexpr int NY = (C / 2) * 8 / 256;    // (channel pair, 8-pair chunk) items per matrix-wave lane
  using S = K3WsSmem;
  __shared__ __attribute__((aligned(16))) S sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  const int N = p.N;
  const size_t ch_stride = size_t(p.B) * N * p.n_pad;
  const uint32_t xo_bytes = uint32_t(p.B) * uint32_t(N) * uint32_t(N) * uint32_t(CZ) * 2u;
  const int G = gridDim.x;
  const int nk = int(blockIdx.x) < p.ntiles ? (p.ntiles - int(blockIdx.x) + G - 1) / G : 0;
  if (nk == 0) return;                      // the whole block: no barrier is left unmatched
  // iterations 0 .. nk do work; both kinds of wave run an even count (one
  // idle iteration at most), so the loops, unrolled by two, have no path that
  // skips half of a body
  const int nit = (nk + 2) & ~1;
  auto tile_at = [&](int k, int& row, int& j0) {
    const int t = int(blockIdx.x) + k * G;
    row = fast_div(t, p.div_nchunk);                     // b * N + i
    j0 = (t - row * p.nchunk) * K3_TP;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  if (wave < 4) {
    // ---- matrix wave: output channels 32 * nb .. 32 * nb + 31 ----
    const int nb = wave;
    const int nrow = 32 * nb + l32;
    bf16x8 wp[KS], wg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      wp[ks] = ld_frag(p.p_out + size_t(nrow) * C + 16 * ks + 8 * lhi);
      wg[ks] = ld_frag(p.g_out + size_t(nrow) * CZ + 16 * ks + 8 * lhi);
    }
    // the output biases go to LDS (read after the prologue's barriers):
    // thread t stages channel t % 128 of p_out_b (t < 128) or g_out_b
    {
      const uint16_t* bsrc = tid < 128 ? p.p_out_b : p.g_out_b;
      (tid < 128 ? sm.bp : sm.bg)[tid & 127] = bsrc ? bf16_to_f32(bsrc[tid & 127]) : 0.0f;
    }
    // accumulator register r holds output channel 32*nb + 8*(r/4) + 4*lhi + r%4:
    // its initial value, the bias, is 4 x 16 bytes of the staged biases
    auto bias_init = [&](const float* bb) {
      f32x16 a;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(bb + 32 * nb + 8 * rg + 4 * lhi);
#pragma unroll
        for (int q = 0; q < 4; ++q) a[4 * rg + q] = v[q];
      }
      return a;
    };
    const auto rsrc_o = __builtin_amdgcn_make_buffer_rsrc(p.out, 0, xo_bytes, 0x00020000);
    constexpr int NST = (K3_TP * CZ / 8) / 256;   // 16-byte out chunks per matrix-wave lane
    auto mma = [&](int b, int mb, f32x16& acc_p, f32x16& acc_g) {
      const int prow = 32 * mb + l32;       // pair this lane feeds as the B operand
      acc_p = bias_init(sm.bp);
      acc_g = bias_init(sm.bg);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 u = ld_frag(sm.u[b] + soff<C>(prow, 2 * ks + lhi));
        const bf16x8 z = ld_frag(sm.z[b] + soff<C>(prow, 2 * ks + lhi));
        acc_p = mfma32x32x16(wp[ks], u, acc_p);
        acc_g = mfma32x32x16(wg[ks], z, acc_g);
      }
    };
    auto gate = [&](int b, int mb, const f32x16& acc_p, const f32x16& acc_g) {
      const int prow = 32 * mb + l32;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = sigmoid_f(acc_g[4 * rg + q]) * acc_p[4 * rg + q];
        const u32x2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(sm.o[b] + ooff<C>(prow, 2 * (4 * nb + rg) + lhi)) = packed;
      }
    };
    // pair-major stores of tile k from out buffer k % 2; for k outside the
    // block's tiles every store goes past the end of out and is dropped
    auto store = [&](int k) {
      const bool valid = k >= 0 && k < nk;
      int row, j0;
      tile_at(valid ? k : 0, row, j0);
      const int so = __builtin_amdgcn_readfirstlane((row * N + j0) * CZ * 2);
      const uint8_t* ob = sm.o[k & 1];
#pragma unroll
      for (int it = 0; it < NST; ++it) {
        const int id = it * 256 + tid;
        const int pr = id / (CZ / 8);
        const int cc = id - pr * (CZ / 8);
        u32x4 v = ld16(ob + pr * (C * 2) + ((cc ^ ((pr & 31) >> 1)) << 4));
        if (pr & 1) v = u32x4{v[2], v[3], v[0], v[1]};
        // a pair past N gets an offset past the end of out (0x80000000 plus a
        // tile base below 2^31 stays below 2^32): the store is dropped
        const uint32_t off = (valid && j0 + pr < N) ? uint32_t(id) * 16u : 0x80000000u;
        buffer_store16(rsrc_o, v, off + uint32_t(so));
      }
    };
    const auto rsrc_y = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.plane_y), 0,
                                                          uint32_t(ch_stride) * uint32_t(C) * 2u, 0x00020000);
    // y item it: channel pair cp = id / 8 (channels 2 cp, 2 cp + 1), 8-pair
    // chunk jc = id % 8 (8 lanes read one channel's 128 bytes)
    uint32_t y_off[NY];
#pragma unroll
    for (int it = 0; it < NY; ++it) {
      const int id = it * 256 + tid;
      y_off[it] = (2u * uint32_t(id >> 3) * uint32_t(ch_stride) + 8u * uint32_t(id & 7)) * 2u;
    }
    const int ych = int(ch_stride) * 2;      // bytes from channel 2 cp to 2 cp + 1
    u32x4 yas[2][NY], ybs[2][NY];            // two register sets: y of tiles of either parity
    auto prefetch_y = [&](int k, auto set) {
      constexpr int e = decltype(set)::value;
      int row, j0;
      tile_at(min(k, nk - 1), row, j0);
      const int sy = __builtin_amdgcn_readfirstlane((row * p.n_pad + j0) * 2);
#pragma unroll
      for (int it = 0; it < NY; ++it) {
        yas[e][it] = buffer_load16(rsrc_y, y_off[it], sy);
        ybs[e][it] = buffer_load16(rsrc_y, y_off[it], sy + ych);
      }
    };
    auto transpose = [&](auto set) {
      constexpr int e = decltype(set)::value;
      const auto& ya = yas[e];
      const auto& yb = ybs[e];
#pragma unroll
      for (int it = 0; it < NY; ++it) {
        const int id = it * 256 + tid;
        const int cp = id >> 3;
        const int jc = id & 7;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r0 = 8 * jc + 2 * q;
          const uint32_t even = __builtin_amdgcn_perm(yb[it][q], ya[it][q], 0x05040100u);   // pair r0
          const uint32_t odd = __builtin_amdgcn_perm(yb[it][q], ya[it][q], 0x07060302u);    // pair r0 + 1
          *reinterpret_cast<uint32_t*>(sm.y + soff<C>(r0, cp >> 2) + 4 * (cp & 3)) = even;
          *reinterpret_cast<uint32_t*>(sm.y + soff<C>(r0 + 1, cp >> 2) + 4 * (cp & 3)) = odd;
        }
      }
    };
    // prologue: the y rows of tile 0, with y of tiles 1 and 2 in flight in
    // the order the loop issues them: a tile's y, one iteration's stores
    // (past the end of out here), the next tile's y (into the set tile 0's
    // transpose has just read)
    prefetch_y(0, I0{});
    prefetch_y(1, I1{});
    store(-2);
    transpose(I0{});
    prefetch_y(2, I0{});
    lds_barrier();                           // y rows of tile 0 (the LayerNorm waves: z of tile 0)
    lds_barrier();                           // u of tile 0
    // iteration k: tile k's matrix work; the y of tile k + 1 (set (k + 1) % 2)
    // transposed, then refilled with tile k + 3
    auto iteration = [&](int k, auto set) {
      const int b = k & 1;
      f32x16 p0, g0, p1, g1;
      if (k < nk) {
        // both gates wait for phase 2: phase 1, with the transpose, is the
        // matrix waves' longer phase
        mma(b, 0, p0, g0);
        mma(b, 1, p1, g1);
      }
      if (k + 1 < nk) transpose(set);
      lds_barrier();
      if (k < nk) {
        gate(b, 0, p0, g0);
        gate(b, 1, p1, g1);
      }
      store(k - 1);
      prefetch_y(k + 3, set);
      lds_barrier();
    };
    for (int k = 0; k < nit; k += 2) {
      iteration(k, I1{});
      iteration(k + 1, I0{});
    }
  } else {
    // ---- LayerNorm wave lw: normalises pairs 16 lw .. 16 lw + 15 ----
    const int lw = wave - 4;
    const int sub = lane & 7;                // sub-lane of a pair (stage-1 mapping)
    const int pl = lane >> 3;                // pair within a pass of 8
    u32x4 inw[NV], inb[NV], outw[NV], outb[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      inw[v] = ld16(p.ln_in_w + 8 * sub + 64 * v);
      inb[v] = ld16(p.ln_in_b + 8 * sub + 64 * v);
      outw[v] = ld16(p.ln_out_w + 8 * sub + 64 * v);
      outb[v] = ld16(p.ln_out_b + 8 * sub + 64 * v);
    }
    const auto rsrc_x = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.x), 0, xo_bytes, 0x00020000);
    // x: pass q, pair 16 lw + 8 q + pl, sub-lane sub
    const uint32_t x_off = (uint32_t(K3W_PAIRS * lw + pl) * CZ + 8u * uint32_t(sub)) * 2u;
    u32x4 xrs[2][2][NV];                     // two register sets
    // pairs past N read the next row's x (or zeros past the end); their
    // outputs are never stored
    auto prefetch_x = [&](int k, auto set) {
      constexpr int e = decltype(set)::value;
      int row, j0;
      tile_at(min(k, nk - 1), row, j0);
      const int sx = __builtin_amdgcn_readfirstlane((row * N + j0) * CZ * 2);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int v = 0; v < NV; ++v) xrs[e][q][v] = buffer_load16(rsrc_x, x_off + 2048u * q + 128u * v, sx);
    };
    // both passes (pairs 16 lw + pl and 16 lw + 8 + pl) in one interleaved
    // LayerNorm: the same bits per pair as layer_norm_row (z_in as stage 1's)
    const int P0 = K3W_PAIRS * lw + pl, P1 = P0 + 8;   // pairs within the tile
    auto ln_in = [&](int b, auto set) {
      constexpr int e = decltype(set)::value;
      u32x4 z0[NV], z1[NV];
      layer_norm_rows2<NV>(xrs[e][0], xrs[e][1], inw, inb, p.eps, z0, z1);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        st16(sm.z[b] + soff<C>(P0, sub + 8 * v), z0[v]);
        st16(sm.z[b] + soff<C>(P1, sub + 8 * v), z1[v]);
      }
    };
    auto ln_out = [&](int b) {
      u32x4 y0[NV], y1[NV], u0[NV], u1[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        y0[v] = ld16(sm.y + soff<C>(P0, sub + 8 * v));
        y1[v] = ld16(sm.y + soff<C>(P1, sub + 8 * v));
      }
      layer_norm_rows2<NV>(y0, y1, outw, outb, p.eps, u0, u1);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        st16(sm.u[b] + soff<C>(P0, sub + 8 * v), u0[v]);
        st16(sm.u[b] + soff<C>(P1, sub + 8 * v), u1[v]);
      }
    };
    // tile k's x lives in register set k % 2
    prefetch_x(0, I0{});
    prefetch_x(1, I1{});
    ln_in(0, I0{});
    prefetch_x(2, I0{});
    lds_barrier();                           // z of tile 0; y rows of tile 0
    ln_out(0);
    lds_barrier();                           // u of tile 0
    // iteration k works on tile k + 1 (set (k + 1) % 2) and refills that set
    // with tile k + 3
    auto iteration = [&](int k, auto set) {
      if (k + 1 < nk) ln_in((k + 1) & 1, set);
      prefetch_x(k + 3, set);
      lds_barrier();
      if (k + 1 < nk) ln_out((k + 1) & 1);
      lds_barrier();
    };
    for (int k = 0; k < nit; k += 2) {
      iteration(k, I1{});
      iteration(k + 1, I0{});
    }
  }
}

}  // namespace

int k3_tiles(int B, int N) { return B * N * ((N + K3_TP - 1) / K3_TP); }

hipError_t launch_k3(const K3Args& a, int grid_x, hipStream_t stream) {
  if (a.c == 128) {
    hipLaunchKernelGGL(k3_epilogue_ws, dim3(grid_x), dim3(K3_THREADS), 0, stream, a);
  } else if (a.c == 256) {
    hipLaunchKernelGGL(k3_epilogue<256>, dim3(grid_x), dim3(K3_THREADS), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace trimul
