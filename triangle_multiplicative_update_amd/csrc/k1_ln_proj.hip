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
// Software pipeline. Each wave splits its multiply into two halves of 32
// pairs and overlaps the matrix cores with the VALU across tile boundaries:
// while the MFMAs of half 1 of tile t run, the wave applies sigmoid * value *
// mask to half 0 of tile t; while the MFMAs of half 0 of tile t+1 run, it
// finishes half 1 of tile t. Between the two, LayerNorm of tile t+1 goes into
// the other z buffer and the x loads of tile t+2 are issued; after the one
// barrier per tile, the block stores tile t-1's staged channel-major outputs
// with 16-byte coalesced writes. z and the mask are double-buffered in LDS,
// the output staging triple-buffered (double for c_z = 256, with a second
// barrier), so no buffer is overwritten while another wave still reads it.

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
  static constexpr int OB = CZ == 128 ? 3 : 2;   // output staging buffers
  uint16_t z[2][K1_TP * ZP];
  uint16_t o[OB][2 * K1_GROUP * OP];
  // mask terms per pair, c_z = 128 form: three buffers, because the gate of
  // a tile's second pair half runs after the tile's barrier and the next
  // tile writes the mask terms of the tile after it before its own barrier
  float mb[3][K1_TP];                      // +inf for m = 0, else 0
  float mi[3][K1_TP];                      // 1 / m, or 1 for m = 0
  float m[2][K1_TP];                       // m (c_z = 256 form: tile-sequential, two suffice)
  float lnw[CZ], lnb[CZ];                  // LayerNorm_in affine, fp32 (c_z = 256 form)
};

template <int CZ>
__global__ __launch_bounds__(K1_THREADS) void k1_ln_proj(const K1Args p) {
  constexpr int NV = CZ / 64;      // 16-byte chunks of a pair row per lane
  constexpr int KS = CZ / 16;      // MFMA k-steps
  // At c_z = 256 the 32 channels' weights alone take 128 registers: the
  // LayerNorm parameters then live in LDS and the biases are kept as one
  // scalar per lane (splat into the accumulator when a chain starts).
  constexpr bool kWide = CZ > 128;
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
  auto splat = [](float v) {
    f32x16 r;
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = v;
    return r;
  };

  // ---- LayerNorm lane mapping: pair `lp`, sub-lane `sub` ----
  const int lp = tid >> 3;
  const int sub = tid & 7;
  u32x4 lnw[NV], lnb[NV];
  if constexpr (kWide) {
    stage_f32(sm.lnw, p.ln_w, CZ);         // read after the prologue's first barrier
    stage_f32(sm.lnb, p.ln_b, CZ);
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      lnw[v] = ld16(p.ln_w + 8 * sub + 64 * v);
      lnb[v] = ld16(p.ln_b + 8 * sub + 64 * v);
    }
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
    if constexpr (kWide) {
      // (zeroing the x of pairs past N keeps this form's register
      // allocation free of spills). A zero row has variance 0: with eps = 0
      // its z would be 0 * inf = NaN, and NaN * (m = 0) stays NaN in the
      // padded plane columns, which every contraction sum reads. Those pairs
      // take eps = 1 instead (z = the LayerNorm bias, finite), so their a and
      // b are +0.0 for any eps >= 0.
      u32x4 xin[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) xin[v] = xok ? xr[v] : u32x4{0, 0, 0, 0};
      layer_norm_row_lds<NV>(xin, sm.lnw, sm.lnb, sub, xok ? p.eps : 1.0f, z);
    } else {
      // pairs past N repeat pair N - 1 of the same plane row: their z is
      // non-finite only where that real pair's is, and then the formula's
      // sums over the row are not finite either
      layer_norm_row<NV>(xr, lnw, lnb, p.eps, z);
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) st16(&sm.z[zb][lp * S::ZP + 8 * sub + 64 * v], z[v]);
    const float m = bf16_bits_late(mraw);  // the 8 lanes of a pair write the same values
    if constexpr (kWide) {
      sm.m[mz][lp] = m;
    } else {
      const bool off = m == 0.0f;
      sm.mb[mz][lp] = off ? __builtin_inff() : 0.0f;
      sm.mi[mz][lp] = off ? 1.0f : __builtin_amdgcn_rcpf(m);
    }
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
          if constexpr (kWide) {
            nv = mfma32x32x16(a, wv[ks], ks == 0 ? splat(bias_vs) : nv);
            ng = mfma32x32x16(a, wg[ks], ks == 0 ? splat(bias_gs) : ng);
          } else {
            nv = mfma32x32x16(a, wv[ks], ks == 0 ? bias_v : nv);
            ng = mfma32x32x16(a, wg[ks], ks == 0 ? bias_g : ng);
          }
        }
      }
      const int m0 = 32 * emb + 8 * rg + 4 * lhi;   // first of 4 consecutive pairs
      float o[4];
      if constexpr (kWide) {
        // (no registers to spare for the two mask terms at c_z = 256)
        const f32x4 mm = *reinterpret_cast<const f32x4*>(&sm.m[emz][m0]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 4 * rg + q;
          o[q] = __builtin_fmaf(sigmoid_f(eg[r]) * ev[r], mm[q], 0.0f);   // +0.0 for m = 0
        }
      } else {
        const f32x4 mb = *reinterpret_cast<const f32x4*>(&sm.mb[emz][m0]);
        const f32x4 mi = *reinterpret_cast<const f32x4*>(&sm.mi[emz][m0]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 4 * rg + q;
          o[q] = gate_masked(eg[r], ev[r], mb[q], mi[q]);
        }
      }
      const u32x2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      *reinterpret_cast<u32x2*>(&sm.o[ob][(plane * K1_GROUP + chs + l32) * S::OP + m0]) = packed;
      if constexpr (kMma && !kWide) {
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
      if constexpr (kWide) {
        nv = mfma32x32x16(a, wv[ks], ks == 0 ? splat(bias_vs) : nv);
        ng = mfma32x32x16(a, wg[ks], ks == 0 ? splat(bias_gs) : ng);
      } else {
        nv = mfma32x32x16(a, wv[ks], ks == 0 ? bias_v : nv);
        ng = mfma32x32x16(a, wg[ks], ks == 0 ? bias_g : ng);
      }
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
  // c_z = 128 keeps the four offsets in registers; c_z = 256 has none to
  // spare and recomputes them per store (as a global store)
  uint32_t st_off[kStoreParts];
  if constexpr (!kWide) {
#pragma unroll
    for (int it = 0; it < kStoreParts; ++it) st_off[it] = lane_off(it);
  }
  auto store_part = [&](int t, int ob, int it) {
    const int row = fast_div(t, p.div_nchunk);
    const int inner0 = (t - row * nchunk) * K1_TP;
    const int srow = (it * K1_THREADS + tid) >> 3;
    const int c16 = tid & 7;
    const int soff = __builtin_amdgcn_readfirstlane((row * p.n_pad + inner0) * 2);
    const u32x4 v = ld16(&sm.o[ob][srow * S::OP + 8 * c16]);
    if constexpr (kWide) {
      const int gch = group * K1_GROUP + (srow & (K1_GROUP - 1));
      st16((it < 2 ? p.plane_a : p.plane_b) + size_t(gch) * ch_stride + size_t(row) * p.n_pad + inner0 + 8 * c16,
           v);
    } else {
      buffer_store16(it < 2 ? rsrc_a : rsrc_b, v, st_off[it] + uint32_t(soff));
    }
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
  if constexpr (kWide) {
    // c_z = 256: the multiply dominates (four times the c = 128 work per
    // pair) and the weights fill half the registers, so the tile runs one
    // pair half at a time (one accumulator pair live): MFMAs then gate for
    // half 0 and half 1, LayerNorm of the next tile, x loads two tiles
    // ahead, one barrier, then the stores of this tile.
    f32x16 av, ag;
    fetch(t);
    lds_barrier();           // LayerNorm parameters staged
    ln_store(0, 0);
    if (t + stride < ntiles) fetch(t + stride);
    no_stores();
    lds_barrier();
    int zb = 0, ob = 0;
    for (; t < ntiles; t += stride) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        mma_only(zb, mb, av, ag);
        half(std::false_type{}, 0, 0, av, ag, av, ag, zb, mb, ob, no_op);
      }
      if (t + stride < ntiles) ln_store(zb ^ 1, zb ^ 1);
      if (t + 2 * stride < ntiles) fetch(t + 2 * stride);
      lds_barrier();
      store(t, ob);
      ob ^= 1;
      zb ^= 1;
    }
  } else {
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
    if constexpr (S::OB == 2) {
      if constexpr (kStore == 1) store(t - stride, prev);
      lds_barrier();
    }
    // next tile's half-0 MFMAs || half 1's gate epilogue (|| the stores)
    const int tp = t - stride, pb = prev;
    auto st = [&](int rg) {
      if constexpr (kStore == 1 && S::OB != 2) {
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
