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
// Software pipeline (c_z = 128, k1_ln_proj). Each wave splits its multiply
// into two halves of 32 pairs and overlaps the matrix cores with the VALU
// across tile boundaries: while the MFMAs of half 1 of tile t run, the wave
// applies sigmoid * value * mask to half 0 of tile t; while the MFMAs of half
// 0 of tile t+1 run, it finishes half 1 of tile t. Between the two, LayerNorm
// of tile t+1 goes into the other z buffer and the x loads of tile t+2 are
// issued; after the one barrier per tile, the block stores tile t-1's staged
// channel-major outputs with 16-byte coalesced writes. z and the mask are
// double-buffered in LDS, the output staging triple-buffered, so no buffer is
// overwritten while another wave still reads it. The c_z = 256 form
// (k1_ln_proj_wide, below) has its own pipeline.

#include <type_traits>

#include "trimul_device.hpp"
#include "trimul_kernels.hpp"

namespace trimul {

namespace {

constexpr int K1_THREADS = 512;

// bf16 1.0 and +0.0: the mask values read for pairs of a call without a mask
// and for pairs past N
__device__ const uint16_t kMaskConst[2] = {0x3F80, 0x0000};
constexpr int K1_TP = 64;          // pairs per tile
constexpr int K1_GROUP = 128;      // channels of a (and of b) per block

template <int CZ>
struct K1Smem {
  static constexpr int ZP = CZ + 8;        // z row pitch (bf16 elements)
  static constexpr int OP = K1_TP + 8;     // staging row pitch
  static constexpr int OB = 3;             // output staging buffers
  uint16_t z[2][K1_TP * ZP];
  uint16_t o[OB][2 * K1_GROUP * OP];
  // mask terms per pair: three buffers, because the gate of a tile's second
  // pair half runs after the tile's barrier and the next tile writes the
  // mask terms of the tile after it before its own barrier
  float mb[3][K1_TP];                      // +inf for m = 0, else 0
  float mi[3][K1_TP];                      // 1 / m, or 1 for m = 0
};

// c_z = 128 form (c_z = 256: k1_ln_proj_wide below)
template <int CZ>
__global__ __launch_bounds__(K1_THREADS) void k1_ln_proj(const K1Args p) {
  static_assert(CZ == 128, "the c_z = 256 form is k1_ln_proj_wide");
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
  // the biases enter as the accumulator input of the first MFMA of a chain
  // (every register of a lane's accumulator belongs to the lane's channel)
  const float bias_vs = p.p_in_b ? bf16_to_f32(p.p_in_b[wrow]) : 0.0f;
  const float bias_gs = p.g_in_b ? bf16_to_f32(p.g_in_b[wrow]) : 0.0f;
  f32x16 bias_v, bias_g;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    bias_v[r] = bias_vs;
    bias_g[r] = bias_gs;
  }

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
  const int nchunk = p.nchunk;
  const int ntiles = p.ntiles;
  const int stride = gridDim.x;
  const size_t ch_stride = size_t(p.B) * N * p.n_pad;
  // no mask: every pair reads the constant 1.0 (index stride 0), so the mask
  // load needs no branch (a branch would force a wait on all memory traffic)
  const uint16_t* mask = p.mask ? p.mask : kMaskConst;
  const int mask_step = p.mask ? 1 : 0;

  // x and mask of this lane's LayerNorm pair in tile t, as loaded; pairs past
  // N read a valid pair's x and the mask constant 0 (their a and b are then
  // +0.0 whatever their z). No instruction uses the loaded values before
  // LayerNorm, so nothing waits for the loads until then.
  u32x4 xr[NV];
  uint16_t mraw = 0;
  bool xok = false;
  auto fetch = [&](int t) {
    const int row = fast_div(t, p.div_nchunk);
    const int inner = (t - row * nchunk) * K1_TP + lp;
    xok = inner < N;
    const int in_c = xok ? inner : N - 1;
    const int bb = fast_div(row, p.div_N);
    const int fixed = row - bb * N;
    // outgoing: pair (b, fixed, inner); incoming: pair (b, inner, fixed)
    const int pi = p.incoming ? (bb * N + in_c) * N + fixed : row * N + in_c;
#pragma unroll
    for (int v = 0; v < NV; ++v) xr[v] = ld16(p.x + size_t(pi) * CZ + 8 * sub + 64 * v);
    mraw = ld_global_u16(xok ? mask + pi * mask_step : kMaskConst + 1);
  };

  // LayerNorm_in of the fetched tile -> z (bf16) in LDS buffer `zb` and the
  // mask terms in mask buffer `mz`. The mask enters the gate as sigmoid(g) v m = v / ((1 + 2^t) / m)
  // with t = -g log2 e: a pair with m = 0 gets t = +inf (so 1 / inf = 0 and
  // the final fma with +0.0 gives exactly +0.0), any other m the factor 1 / m
  // in the denominator (1 / 1 = 1 exactly, so m = 1 costs no rounding).
  auto ln_store = [&](int zb, int mz) {
    u32x4 z[NV];
    // pairs past N repeat pair N - 1 of the same plane row: their z is
    // non-finite only where that real pair's is, and then the formula's
    // sums over the row are not finite either
    layer_norm_row<NV>(xr, lnw, lnb, p.eps, z);
#pragma unroll
    for (int v = 0; v < NV; ++v) st16(&sm.z[zb][lp * S::ZP + 8 * sub + 64 * v], z[v]);
    const float m = bf16_bits_late(mraw);  // the 8 lanes of a pair write the same values
    const bool off = m == 0.0f;
    sm.mb[mz][lp] = off ? __builtin_inff() : 0.0f;
    sm.mi[mz][lp] = off ? 1.0f : __builtin_amdgcn_rcpf(m);
  };

  // One overlapped half step. With DO_MMA: the 2 * KS MFMAs of pair half
  // `mb` of the tile in z buffer `zb` into (nv, ng). Interleaved with them:
  // sigmoid(eg) * ev * mask for pair half `emb` of the tile whose mask terms
  // are in mask buffer `emz`, rounded to bf16 and staged channel-major in output buffer
  // `ob`. The accumulator layout puts 4 consecutive pairs of one channel in
  // each register group, i.e. 8 contiguous bytes of a staging row.
  auto half = [&](auto do_mma, int zb, int mb, f32x16& nv, f32x16& ng, const f32x16& ev,
                  const f32x16& eg, int emz, int emb, int ob, auto&& each_rg) {
    constexpr bool kMma = decltype(do_mma)::value;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      each_rg(rg);
      if constexpr (kMma) {
#pragma unroll
        for (int kk = 0; kk < KS / 4; ++kk) {
          const int ks = rg * (KS / 4) + kk;
          const bf16x8 a = ld_frag(&sm.z[zb][(32 * mb + l32) * S::ZP + 16 * ks + 8 * lhi]);
          nv = mfma32x32x16(a, wv[ks], ks == 0 ? bias_v : nv);
          ng = mfma32x32x16(a, wg[ks], ks == 0 ? bias_g : ng);
        }
      }
      const int m0 = 32 * emb + 8 * rg + 4 * lhi;   // first of 4 consecutive pairs
      float o[4];
      const f32x4 mb = *reinterpret_cast<const f32x4*>(&sm.mb[emz][m0]);
      const f32x4 mi = *reinterpret_cast<const f32x4*>(&sm.mi[emz][m0]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * rg + q;
        o[q] = gate_masked(eg[r], ev[r], mb[q], mi[q]);
      }
      const u32x2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      *reinterpret_cast<u32x2*>(&sm.o[ob][(plane * K1_GROUP + chs + l32) * S::OP + m0]) = packed;
      if constexpr (kMma) {
        // scheduling hint for the register group: its four LDS reads first,
        // then each MFMA followed by three VALU instructions (measured best
        // of 3, 5 and 8; the MFMAs otherwise issue in a burst)
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      }
    }
  };

  // the MFMAs of a half step on their own (first tile of the block)
  auto mma_only = [&](int zb, int mb, f32x16& nv, f32x16& ng) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = ld_frag(&sm.z[zb][(32 * mb + l32) * S::ZP + 16 * ks + 8 * lhi]);
      nv = mfma32x32x16(a, wv[ks], ks == 0 ? bias_v : nv);
      ng = mfma32x32x16(a, wg[ks], ks == 0 ? bias_g : ng);
    }
  };

  // coalesced plane stores of tile t from output buffer `ob`: 256 rows
  // (128 a + 128 b channels) x 64 pairs, one 16-byte chunk per thread and
  // part `it` (0..3); n_pad is a multiple of 64, so every chunk of the tile
  // lies inside its row
  // Buffer stores: a lane's byte offset inside a tile (channel row and
  // chunk) is the same for every tile and sits in a register; the tile's
  // (row, first pair) offset is uniform and is added to it per store. Every
  // plane is below 2^31 bytes (the extent rule), so 32-bit offsets suffice.
  constexpr int kStoreParts = (2 * K1_GROUP * K1_TP / 8) / K1_THREADS;
  static_assert(kStoreParts == 4 && K1_THREADS / 8 * 2 == K1_GROUP, "parts 0-1: plane a, 2-3: plane b");
  const uint32_t plane_bytes = uint32_t(ch_stride) * uint32_t(p.c) * 2u;
  const auto rsrc_a = __builtin_amdgcn_make_buffer_rsrc(p.plane_a, 0, plane_bytes, 0x00020000);
  const auto rsrc_b = __builtin_amdgcn_make_buffer_rsrc(p.plane_b, 0, plane_bytes, 0x00020000);
  auto lane_off = [&](int it) {
    const int srow = (it * K1_THREADS + tid) >> 3;   // staging row: plane * 128 + channel
    const int gch = group * K1_GROUP + (srow & (K1_GROUP - 1));
    return (uint32_t(gch) * uint32_t(ch_stride) + 8u * uint32_t(tid & 7)) * 2u;
  };
  uint32_t st_off[kStoreParts];
#pragma unroll
  for (int it = 0; it < kStoreParts; ++it) st_off[it] = lane_off(it);
  auto store_part = [&](int t, int ob, int it) {
    const int row = fast_div(t, p.div_nchunk);
    const int inner0 = (t - row * nchunk) * K1_TP;
    const int srow = (it * K1_THREADS + tid) >> 3;
    const int c16 = tid & 7;
    const int soff = __builtin_amdgcn_readfirstlane((row * p.n_pad + inner0) * 2);
    const u32x4 v = ld16(&sm.o[ob][srow * S::OP + 8 * c16]);
    buffer_store16(it < 2 ? rsrc_a : rsrc_b, v, st_off[it] + uint32_t(soff));
  };
  auto store = [&](int t, int ob) {
#pragma unroll
    for (int it = 0; it < kStoreParts; ++it) store_part(t, ob, it);
  };
  // Vector-memory operations retire in issue order, so a wait for the x and
  // mask loads of a later tile is a count of what was issued after them: the
  // previous tile's plane stores. The compiler takes that count once per loop
  // and merges the paths into the loop, so every path must issue the same
  // number of stores after the loads, or the wait falls back to draining the
  // stores. Where there is no previous tile, these stores stand in: their
  // offset lies past the end of plane a, so the hardware drops them.
  // (distinct offsets, so the compiler does not merge them)
  auto no_store = [&](int it) { __builtin_amdgcn_raw_buffer_store_b32(0u, rsrc_a, 0x80000000u + 16u * it, 0, 0); };
  auto no_stores = [&]() {
#pragma unroll
    for (int it = 0; it < kStoreParts; ++it) no_store(it);
  };
  auto no_op = [](int) {};

  int t = blockIdx.x;
  if (t >= ntiles) return;
  f32x16 v0, g0, v1, g1;   // accumulators of pair halves 0 and 1

  // prologue: LayerNorm of the first tile, x of the second in flight, the
  // MFMAs of the first tile's half 0
  fetch(t);
  ln_store(0, 0);
  if (t + stride < ntiles) fetch(t + stride);
  no_stores();
  lds_barrier();
  mma_only(0, 0, v0, g0);

  // One tile t with z buffer zb, output buffer ob; `prev` names the output
  // buffer of the block's previous tile, still to be stored. kStore: 0 = no
  // previous tile, 1 = one store part per register group of the overlapped
  // half step (the stores trickle out between the MFMAs instead of stalling
  // every wave at once), 2 = whole store if prev >= 0 (the last tiles).
  int zb = 0, ob = 0, prev = -1, mz = 0;   // mz: mask buffer of tile t
  auto tile = [&](auto store_mode, auto has_next, auto has_next2) {
    constexpr int kStore = decltype(store_mode)::value;
    constexpr bool kNext = decltype(has_next)::value;
    constexpr bool kNext2 = decltype(has_next2)::value;
    // half 1's MFMAs || half 0's gate epilogue
    const int mz_next = mz == 2 ? 0 : mz + 1;
    half(std::true_type{}, zb, 1, v1, g1, v0, g0, mz, 0, ob, no_op);
    if constexpr (kNext) ln_store(zb ^ 1, mz_next);
    if constexpr (kNext2) fetch(t + 2 * stride);
    lds_barrier();
    if constexpr (kStore == 2) {
      if (prev >= 0) store(t - stride, prev);
    }
    // next tile's half-0 MFMAs || half 1's gate epilogue (|| the stores)
    const int tp = t - stride, pb = prev;
    auto st = [&](int rg) {
      if constexpr (kStore == 1) {
        if (rg < kStoreParts) store_part(tp, pb, rg);
      } else if constexpr (kStore == 0) {
        if (rg < kStoreParts) no_store(rg);
      }
    };
    if constexpr (kNext) half(std::true_type{}, zb ^ 1, 0, v0, g0, v1, g1, mz, 1, ob, st);
    else half(std::false_type{}, 0, 0, v0, g0, v1, g1, mz, 1, ob, st);
    prev = ob;
    ob = (ob + 1 == S::OB) ? 0 : ob + 1;
    zb ^= 1;
    mz = mz_next;
    t += stride;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // steady state: every part unconditional
  if (t + 2 * stride < ntiles) tile(I0{}, std::true_type{}, std::true_type{});
  while (t + 2 * stride < ntiles) tile(I1{}, std::true_type{}, std::true_type{});
  if (t + stride < ntiles) tile(I2{}, std::true_type{}, std::false_type{});
  tile(I2{}, std::false_type{}, std::false_type{});
  lds_barrier();
  store(t - stride, prev);
}


// ---------------------------------------------------------------------------
// c_z = 256 form. The 32 channels' value and gate weights of a wave fill 128
// registers, so a tile's accumulators cannot be held whole. The multiply
// therefore runs as 16 x 16 x 32 MFMAs over four pair groups of 16 pairs:
// the accumulators of one group (2 channel blocks x value, gate) are 16
// registers, and the gate of group g - 1 runs on the VALU while the matrix
// cores work on group g (two accumulator sets live, as many registers as one
// 32-pair half of 32 x 32 MFMAs). The LayerNorm of the next tile is split
// into its three passes (mean, variance, normalise) and spread over three of
// the four group steps, so every step has vector work beside the MFMAs.
//
// x travels by direct global -> LDS loads into a ring of three 32 KB pair
// tiles; LayerNorm_in then runs in place, so the tile turns from x into z
// where it lies. Tile k of the block is loaded at the start of step k - 2,
// normalised during step k - 1 and multiplied during step k. Every wave
// loads the eight pair rows its own lanes normalise, so the only wait before
// the LayerNorm is on the wave's own loads; one barrier per tile publishes z.
// The gated outputs go from registers to the planes as 8-byte stores (four
// pairs of one channel per lane, 32 contiguous bytes per channel and group);
// the four groups of a tile fill each 128-byte line of a channel row.
//
// Pair tile layout: row r (pair) of 512 bytes, 16-byte chunk c at slot
// c ^ wide_swz(r). Under the LDS bank model this keeps both the LayerNorm
// rows (8 lanes x 16 bytes per row) and the MFMA A-fragment reads (16 rows at
// one chunk, the next 16 lanes at the next chunk) conflict-free.
__device__ __forceinline__ int wide_swz(int r) {
  return ((r & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2) | (((r >> 1) & 1) << 3);
}

struct K1WideSmem {
  static constexpr int kTileBytes = K1_TP * 256 * 2;
  uint8_t xz[3][kTileBytes];               // x, then z in place
  float mb[3][K1_TP];                      // mask terms, as in the c_z = 128 form
  float mi[3][K1_TP];
  float lnw[256], lnb[256];                // LayerNorm_in affine, fp32
};

__global__ __launch_bounds__(K1_THREADS) void k1_ln_proj_wide(const K1Args p) {
  constexpr int CZ = 256;
  constexpr int NV = CZ / 64;      // LayerNorm chunks per lane
  constexpr int KS = CZ / 32;      // MFMA k-steps
  constexpr int NLD = K1WideSmem::kTileBytes / 1024 / 8;   // 1 KB direct loads per wave and tile
  static_assert(NLD == 4, "a wave loads the 8 pair rows of its LayerNorm lanes");
  // vector-memory operations of a tile step, in issue order: the mask load of
  // the next tile, NLD x loads of the tile after it, 2 plane stores per group
  constexpr int kStoresPerStep = 8;
  __shared__ __attribute__((aligned(16))) K1WideSmem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int group = blockIdx.y;

  // ---- weights: plane (wave / 4), 32 channels as two blocks of 16 ----
  const int plane = wave >> 2;
  const int chs = 32 * (wave & 3);
  bf16x8 wv[2][KS], wg[2][KS];
  float bias_v[2], bias_g[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int wrow = plane * p.c + group * K1_GROUP + chs + 16 * cb + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      wv[cb][ks] = ld_frag(p.p_in + size_t(wrow) * CZ + 32 * ks + 8 * q4);
      wg[cb][ks] = ld_frag(p.g_in + size_t(wrow) * CZ + 32 * ks + 8 * q4);
    }
    bias_v[cb] = p.p_in_b ? bf16_to_f32(p.p_in_b[wrow]) : 0.0f;
    bias_g[cb] = p.g_in_b ? bf16_to_f32(p.g_in_b[wrow]) : 0.0f;
  }
  stage_f32(sm.lnw, p.ln_w, CZ);
  stage_f32(sm.lnb, p.ln_b, CZ);

  const int N = p.N;
  const int G = __builtin_amdgcn_readfirstlane(int(gridDim.x));
  const int nk = __builtin_amdgcn_readfirstlane(
      int(blockIdx.x) < p.ntiles ? (p.ntiles - int(blockIdx.x) + G - 1) / G : 0);
  if (nk == 0) return;                     // the whole block: no barrier is left unmatched
  // Tile k of this block covers pairs inner0 .. inner0 + 63 of plane row
  // b * N + i; pair j of it is x row  base + min(inner0 + j, N - 1) * step:
  // outgoing (b, i, j): base = (b N + i) N, step 1; incoming (b, j, i):
  // base = b N N + i, step N. All uniform.
  struct Tile {
    int inner0;
    int base;
  };
  const int step = p.incoming ? N : 1;
  auto tile_at = [&](int k) {
    const int t = int(blockIdx.x) + k * G;
    const int row = fast_div(t, p.div_nchunk);
    const int bb = fast_div(row, p.div_N);
    const int fixed = row - bb * N;
    Tile tl;
    tl.inner0 = (t - row * p.nchunk) * K1_TP;
    tl.base = p.incoming ? bb * N * N + fixed : row * N;
    tl.inner0 = __builtin_amdgcn_readfirstlane(tl.inner0);
    tl.base = __builtin_amdgcn_readfirstlane(tl.base);
    return tl;
  };
  auto pair_index = [&](const Tile& tl, int j) { return tl.base + min(tl.inner0 + j, N - 1) * step; };

  // x of tile k -> ring slot b: wave w loads pair rows 8w .. 8w + 7, chunk c
  // of row r to slot c ^ wide_swz(r); a pair past N reads pair N - 1. Byte
  // offsets fit 32 bits (x is below 2^31 bytes).
  // Load q of wave w fills tile slots (4w + q) * 64 + lane: pair row
  // pr = 8w + 2q + lane / 32, slot lane % 32. wide_swz(pr) depends on q only
  // through q & 1 (bit 3 of the row), so two chunk offsets serve all four.
  const char* xbytes = reinterpret_cast<const char*>(p.x);
  const int hi = lane >> 5;
  const uint32_t xcol0 = uint32_t(((lane & 31) ^ wide_swz(8 * wave + hi)) << 4);       // q even
  const uint32_t xcol1 = uint32_t(((lane & 31) ^ wide_swz(8 * wave + 2 + hi)) << 4);   // q odd
  auto load_x = [&](int k, int b) {
    const Tile tl = tile_at(k);
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int pr = 8 * wave + 2 * q + hi;
      const uint32_t off = uint32_t(pair_index(tl, pr)) * uint32_t(CZ * 2) + ((q & 1) ? xcol1 : xcol0);
      load_lds16_asm(xbytes, off, sm.xz[b] + (wave * NLD + q) * 1024);
    }
  };

  // LayerNorm lane mapping: pair lp, sub-lane sub (8 lanes per pair)
  const int lp = tid >> 3;
  const int sub = tid & 7;
  const int lswz = wide_swz(lp);
  const uint16_t* mask = p.mask ? p.mask : kMaskConst;
  const int mask_step = p.mask ? 1 : 0;
  auto load_mask = [&](int k) -> uint16_t {
    const Tile tl = tile_at(k);
    const int pi = pair_index(tl, lp);
    return ld_global_u16(tl.inner0 + lp < N ? mask + pi * mask_step : kMaskConst + 1);
  };
  // chunk c of this lane's pair row in slot b: (sub + 8c) ^ lswz is
  // (sub ^ (lswz & 7)) + 8 (c ^ (lswz >> 3)), so chunks c and c + 2 are 256
  // bytes apart and two lane offsets serve all four
  const uint32_t lrow0 = uint32_t(lp * 512 + (((sub ^ (lswz & 7)) + 8 * ((lswz >> 3) & 1)) << 4));
  const uint32_t lrow1 = lrow0 ^ 128u;
  auto row_chunk = [&](int b, int c) -> uint8_t* {
    return sm.xz[b] + ((c & 1) ? lrow1 : lrow0) + 256 * (c >> 1);
  };

  // ---- MFMAs of pair group pg of the z tile in slot b ----
  // rows 16 pg + l16 share the swizzle of l16; (4 ks + q4) ^ aswz is
  // 16 (ks >> 2) + ((4 (ks & 3) + q4) ^ aswz): four lane offsets serve the
  // eight k-steps
  const int aswz = wide_swz(l16);
  uint32_t aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aoff[j] = uint32_t(l16 * 512 + (((4 * j + q4) ^ aswz) << 4));
  auto afrag = [&](int b, int pg, int ks) {
    return ld_frag(sm.xz[b] + aoff[ks & 3] + 256 * (ks >> 2) + 8192 * pg);
  };
  auto mfma4 = [&](const bf16x8& a, int ks, f32x4 (&acc)[4]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const f32x4 iv = {bias_v[cb], bias_v[cb], bias_v[cb], bias_v[cb]};
      const f32x4 ig = {bias_g[cb], bias_g[cb], bias_g[cb], bias_g[cb]};
      acc[2 * cb] = mfma16x16x32(a, wv[cb][ks], ks == 0 ? iv : acc[2 * cb]);
      acc[2 * cb + 1] = mfma16x16x32(a, wg[cb][ks], ks == 0 ? ig : acc[2 * cb + 1]);
    }
  };

  // ---- plane stores ----
  // tile_off: byte offset of the tile's first pair in a channel row, or
  // kNoTile (past the end of every plane: the hardware drops the store)
  constexpr uint32_t kNoTile = 0x80000000u;
  const uint32_t ch_elems = uint32_t(size_t(p.B) * N * p.n_pad);
  const uint32_t plane_bytes = ch_elems * uint32_t(p.c) * 2u;
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(plane ? p.plane_b : p.plane_a, 0, plane_bytes, 0x00020000);
  uint32_t lane_off[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const uint32_t gch = uint32_t(group * K1_GROUP + chs + 16 * cb + l16);
    lane_off[cb] = (gch * ch_elems + 4u * uint32_t(q4)) * 2u;
  }
  auto tile_off_of = [&](int k) {
    const int t = int(blockIdx.x) + k * G;
    const int row = fast_div(t, p.div_nchunk);
    const int inner0 = (t - row * p.nchunk) * K1_TP;
    return uint32_t(__builtin_amdgcn_readfirstlane((row * p.n_pad + inner0) * 2));
  };

  // One group step: the MFMAs of group pg of the tile in slot b into `acc`,
  // and, one output per k-step between them, the gate of group gpg (mask
  // terms in slot gb) from `eacc`, stored at tile offset goff. ln(ks) adds
  // this step's share of the next tile's LayerNorm after k-step ks. The
  // scheduling barriers keep each k-step's work together, so the registers
  // live at any point are those of one k-step.
  auto group_step = [&](int b, int pg, f32x4 (&acc)[4], const f32x4 (&eacc)[4], int gb, int gpg, uint32_t goff,
                        auto&& ln) {
    const int m0 = 16 * gpg + 4 * q4;      // first of this lane's 4 consecutive gated pairs
    const f32x4 mb = *reinterpret_cast<const f32x4*>(&sm.mb[gb][m0]);
    const f32x4 mi = *reinterpret_cast<const f32x4*>(&sm.mi[gb][m0]);
    bf16x8 a = afrag(b, pg, 0);
    float o[4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 an = afrag(b, pg, ks + 1 < KS ? ks + 1 : ks);
      mfma4(a, ks, acc);
      const int cb = ks >> 2, i = ks & 3;
      o[i] = gate_masked(eacc[2 * cb + 1][i], eacc[2 * cb][i], mb[i], mi[i]);
      if (i == 3) {
        const u32x2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        buffer_store8(rsrc, packed, lane_off[cb] + goff + uint32_t(32 * gpg));
      }
      ln(ks);
      a = an;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- LayerNorm of the next tile, a chunk of a pass per two k-steps ----
  float ln_sp[4], ln_mu = 0.0f, ln_rs = 0.0f;
  u32x4 ln_x;
  auto ln_pass1 = [&](int b) {
    return [&, b](int ks) {
      const int c = ks >> 1;
      if ((ks & 1) == 0) ln_x = ld16(row_chunk(b, c));
      else ln_sum_chunk(ln_sp, ln_x, c);
      if (ks == KS - 1) ln_mu = ln_mean_of<NV>(ln_sp);
    };
  };
  auto ln_pass2 = [&](int b) {
    return [&, b](int ks) {
      const int c = ks >> 1;
      if ((ks & 1) == 0) ln_x = ld16(row_chunk(b, c));
      else ln_sq_chunk(ln_sp, ln_x, c, ln_mu);
      if (ks == KS - 1) ln_rs = ln_rstd_of<NV>(ln_sp, p.eps);
    };
  };
  // pass 3, chunks c0 and c0 + 1: read at k-steps 0 and 4, written at 1 and 5
  float ln_w[8], ln_b[8];
  auto ln_pass3 = [&](int b, int c0) {
    return [&, b, c0](int ks) {
      const int c = c0 + (ks >> 2);
      if ((ks & 3) == 0) {
        ln_x = ld16(row_chunk(b, c));
        lds_affine8(sm.lnw, sm.lnb, sub, c, ln_w, ln_b);
      } else if ((ks & 3) == 1) {
        st16(row_chunk(b, c), ln_apply_chunk(ln_x, ln_mu, ln_rs, ln_w, ln_b));
      }
    };
  };
  auto ln_mask = [&](int b, uint16_t mraw) {
    const float m = bf16_bits_late(mraw);   // the 8 lanes of a pair write the same values
    const bool off = m == 0.0f;
    sm.mb[b][lp] = off ? __builtin_inff() : 0.0f;
    sm.mi[b][lp] = off ? 1.0f : __builtin_amdgcn_rcpf(m);
  };
  auto no_ln = [](int) {};

  // ---- prologue: tile 0 loaded and normalised, tile 1 loaded ----
  uint16_t mraw = load_mask(0);
  load_x(0, 0);
  load_x(nk > 1 ? 1 : 0, 1);
  // stand-ins for the plane stores of a step before tile 1's loads are waited
  // for (their offset is past the end of the plane: dropped), so that the
  // wait below counts the same operations in every step
#pragma unroll
  for (int i = 0; i < kStoresPerStep; ++i)
    __builtin_amdgcn_raw_buffer_store_b32(0u, rsrc, kNoTile + 16u * uint32_t(i), 0, 0);
  lds_barrier();                            // LayerNorm affine staged
  wait_vm<NLD + kStoresPerStep>();          // this wave's rows of tile 0 have landed
  {
    u32x4 xr[NV], z[NV];
#pragma unroll
    for (int c = 0; c < NV; ++c) xr[c] = ld16(row_chunk(0, c));
    const float mu = ln_mean<NV>(xr);
    ln_apply<NV>(xr, mu, ln_rstd<NV>(xr, mu, p.eps),
                 [&](int c, float (&w8)[8], float (&b8)[8]) { lds_affine8(sm.lnw, sm.lnb, sub, c, w8, b8); }, z);
#pragma unroll
    for (int c = 0; c < NV; ++c) st16(row_chunk(0, c), z[c]);
    ln_mask(0, mraw);
  }
  lds_barrier();

  f32x4 acc_a[4], acc_b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc_b[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t prev_off = kNoTile;              // tile offset of the previous tile (its group 3 is gated late)
  int bprev = 2, b0 = 0, b1 = 1, b2 = 2;    // ring slots of tiles k - 1, k, k + 1, k + 2
  for (int k = 0; k < nk; ++k) {
    const uint32_t cur_off = tile_off_of(k);
    // the next tile's mask, the x of the tile after it (tiles past the
    // block's last reload the current one: the slot is free, nothing reads it)
    mraw = load_mask(k + 1 < nk ? k + 1 : k);
    load_x(k + 2 < nk ? k + 2 : k, b2);
    // tile k + 1's x was loaded one step ago; issued since: that step's
    // stores, this step's mask load and x loads
    wait_vm<kStoresPerStep + 1 + NLD>();
    group_step(b0, 0, acc_a, acc_b, bprev, 3, prev_off, ln_pass1(b1));
    group_step(b0, 1, acc_b, acc_a, b0, 0, cur_off, ln_pass2(b1));
    group_step(b0, 2, acc_a, acc_b, b0, 1, cur_off, ln_pass3(b1, 0));
    group_step(b0, 3, acc_b, acc_a, b0, 2, cur_off, ln_pass3(b1, 2));
    ln_mask(b1, mraw);
    lds_barrier();                          // z of tile k + 1 complete; slot b0 free after this step
    prev_off = cur_off;
    bprev = b0;
    b0 = b1;
    b1 = b2;
    b2 = bprev;
  }
  // the last tile's group 3 (no MFMAs beside it)
  {
    const int m0 = 48 + 4 * q4;
    const f32x4 mb = *reinterpret_cast<const f32x4*>(&sm.mb[bprev][m0]);
    const f32x4 mi = *reinterpret_cast<const f32x4*>(&sm.mi[bprev][m0]);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = gate_masked(acc_b[2 * cb + 1][i], acc_b[2 * cb][i], mb[i], mi[i]);
      const u32x2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      buffer_store8(rsrc, packed, lane_off[cb] + prev_off + 96u);
    }
  }
}

}  // namespace

hipError_t launch_k1(const K1Args& a, int grid_x, hipStream_t stream) {
  const dim3 grid(grid_x, a.c / K1_GROUP);
  if (a.c_z == 128) {
    hipLaunchKernelGGL(k1_ln_proj<128>, grid, dim3(K1_THREADS), 0, stream, a);
  } else if (a.c_z == 256) {
    hipLaunchKernelGGL(k1_ln_proj_wide, grid, dim3(K1_THREADS), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int k1_tiles(int B, int N) { return B * N * ((N + K1_TP - 1) / K1_TP); }

}  // namespace trimul
