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
// are persistent. Two forms: at c = 128 the waves specialise
// (k3_epilogue_ws: four matrix waves, four LayerNorm waves, one of each per
// SIMD); at c = 256, where every wave must hold 32 output channels' weights,
// the waves specialise by phase instead (k3_epilogue_h256: each wave runs its
// share of the MFMAs in one phase and LayerNorm work in the other, the two
// waves of a SIMD in opposite phases, over half tiles of 32 pairs). Both
// transpose y to pair-major LDS rows two channels per dword, run LayerNorm_in
// with the stage-1 lane mapping (so z_in is bit-identical) and LayerNorm_out,
// compute the value and gate with MFMA 32x32x16 as D[out channel][pair]
// (weights as the A operand, held in registers), and stage sigmoid * value
// as bf16 in LDS [pair][channel] for 16-byte coalesced stores. The pair-major
// tiles use XOR slot swizzles (lds_swz for 256-byte rows, swz32 for the
// 512-byte rows of a half tile); the out staging tile has its own
// 8-byte-unit swizzle (ooff); all conflict-free for their accesses under
// gfx950's LDS bank model.

#include "trimul_device.hpp"
#include "trimul_kernels.hpp"

namespace trimul {

namespace {

constexpr int K3_THREADS = 512;
constexpr int K3_TP = 64;

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

// ---------------------------------------------------------------------------
// c = 256, phase-specialised form. The unit of work is a half tile of 32
// pairs (b, i, j0 .. j0 + 31), the two halves of each 64-pair tile one after
// the other. Every wave holds the p_out and g_out rows of its 32 output
// channels (128 registers) and runs its share of every half tile's MFMAs, but
// the two waves of a SIMD do so in opposite phases, each running vector-ALU
// work while the other's matrix cores run (MFMA and vector issue share a
// SIMD, so the waves' instruction streams, not their phases, set the time).
// Iteration h (half tile h's MFMAs, buffers b = h % 2):
//   phase 1: waves 0-3 run their channel blocks of h (u[b], z[b] -> o[b]);
//            between the MFMAs of the first k-steps they transpose their
//            64-channel slices of the y of half tile h + 1 (ys -> u[b^1]),
//            and after the second half of a tile, issue the next tile's y
//            loads over the remaining k-steps, so that the issue waits
//            overlap the MFMAs. Waves 4-7 run LayerNorm_in of h + 1 on their
//            8 pairs (xs -> z[b^1], the stage-1 lane mapping), issuing the x
//            loads of h + 2 into xs once the rows are in registers.
//   phase 2: waves 4-7 run their channel blocks of h (-> o[b]); waves 0-3
//            run LayerNorm_out of h + 1 in place on their 8 pairs of u[b^1]
//            and store half tile h - 1 from o[b^1].
// y is staged per 64-pair tile as full 128-byte lines (both halves at once;
// loading each half's 64 bytes separately doubles the requests and stalls
// the issue), x per half tile. Each kind of wave loads only the LDS bytes it
// reads itself, so its loads need no barrier, only its own wait count: waves
// 4-7 issue nothing but x loads (wait for all), waves 0-3 a tile's y loads
// and then one iteration's stores (wait for all but those stores). Stores of
// half tiles that do not exist go past the end of out, so every iteration
// issues the same stores.
constexpr int K3H_TP = 32;                 // pairs per half tile
constexpr int K3H_PF = 2;                  // fragment ring depth (k-steps in flight + 1)

// Pair rows of 512 bytes (256 bf16 channels) of a 32-row tile: 16-byte slot s
// of row r at slot s ^ swz32(r), row bits XOR-ed in as bit 0 -> 1, bit 1 -> 8,
// bit 3 -> 4, bit 4 -> 10 (bit 2 -> 0). Under the LDS bank model this keeps
// the MFMA fragment reads (32 consecutive rows at one slot, the upper 32 lanes
// at the next), the LayerNorm rows (8 lanes x 16 bytes per row, 8 rows) and
// the transposing 4-byte writes (4 rows {8 j + e} x 16 consecutive dwords)
// conflict-free.
__device__ __forceinline__ int swz32(int r) {
  return ((r & 1) ? 1 : 0) ^ ((r & 2) ? 8 : 0) ^ ((r & 8) ? 4 : 0) ^ ((r & 16) ? 10 : 0);
}
__device__ __forceinline__ int soff32(int r, int slot) { return r * 512 + ((slot ^ swz32(r)) << 4); }

struct K3HSmem {
  static constexpr int TB = K3H_TP * 512;  // one 32-pair tile of 512-byte rows
  uint8_t u[2][TB];                        // transposed y rows, then u in place
  uint8_t z[2][TB];                        // z_in
  uint8_t o[2][TB];                        // out staging
  uint8_t ys[2 * TB];                      // y of a whole 64-pair tile as loaded (see load_y)
  uint8_t xs[TB];                          // x of a half tile as loaded
  float inw[256], inb[256], outw[256], outb[256], bp[256], bg[256];
};

__global__ __launch_bounds__(K3_THREADS) void k3_epilogue_h256(const K3Args p) {
  constexpr int C = 256, CZ = 256;
  constexpr int NV = C / 64;               // LayerNorm chunks per lane
  constexpr int KS = C / 16;               // MFMA k-steps
  constexpr int NLD = 4;                   // 1 KB x loads per wave of waves 4-7 per half tile
  constexpr int NLY = 8;                   // 1 KB y loads per wave of waves 0-3 per 64-pair tile
  constexpr int NST = 4;                   // 16-byte out stores per lane of waves 0-3 per half tile
  static_assert(NLD * 4 * 1024 == K3HSmem::TB && NST * 256 * 16 == K3HSmem::TB, "one tile per wave kind");
  static_assert(NLY * 4 * 1024 == sizeof(K3HSmem::ys), "y of a 64-pair tile");
  using S = K3HSmem;
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
  const int nh = 2 * nk;                    // half tiles of this block
  auto half_at = [&](int h, int& row, int& j0) {
    const int t = int(blockIdx.x) + (h >> 1) * G;
    row = fast_div(t, p.div_nchunk);                     // b * N + i
    j0 = (t - row * p.nchunk) * K3_TP + K3H_TP * (h & 1);
  };

  // ---- this wave's output channels 32 nb .. 32 nb + 31 ----
  const int nb = wave;
  const int nrow = 32 * nb + l32;          // weight row (output channel) this lane feeds
  bf16x8 wp[KS], wg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    wp[ks] = ld_frag(p.p_out + size_t(nrow) * C + 16 * ks + 8 * lhi);
    wg[ks] = ld_frag(p.g_out + size_t(nrow) * CZ + 16 * ks + 8 * lhi);
  }
  stage_f32(sm.inw, p.ln_in_w, CZ);
  stage_f32(sm.inb, p.ln_in_b, CZ);
  stage_f32(sm.outw, p.ln_out_w, C);
  stage_f32(sm.outb, p.ln_out_b, C);
  stage_f32(sm.bp, p.p_out_b, CZ);
  stage_f32(sm.bg, p.g_out_b, CZ);

  // output projection and gate of half tile in buffers b for this wave's 32
  // channels: D[out channel][pair], then sigmoid * value as bf16 into o[b]
  auto mma_gate = [&](int b, auto&& at_kstep) {
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
    // soff32(l32, 2 ks + lhi) = fbase + 256 (ks >> 3) + 32 ((ks & 7) ^ ft)
    const int fs = swz32(l32);
    int fbase = l32 * 512 + ((lhi ^ (fs & 1)) << 4);
    int ft = fs >> 1;
    asm volatile("" : "+v"(fbase), "+v"(ft));
    auto faddr = [&](int ks) { return fbase + 256 * (ks >> 3) + ((((ks & 7) ^ ft)) << 5); };
    const uint8_t* ub = sm.u[b];
    const uint8_t* zb = sm.z[b];
    // the fragments of k-step ks + PF - 1 are read before the MFMAs of ks: the
    // other wave of the SIMD runs vector work, not MFMAs, while this one waits
    bf16x8 uf[K3H_PF], zf[K3H_PF];
#pragma unroll
    for (int i = 0; i < K3H_PF - 1; ++i) {
      uf[i] = ld_frag(ub + faddr(i));
      zf[i] = ld_frag(zb + faddr(i));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + K3H_PF - 1 < KS) {
        const int a = faddr(ks + K3H_PF - 1);
        uf[(ks + K3H_PF - 1) % K3H_PF] = ld_frag(ub + a);
        zf[(ks + K3H_PF - 1) % K3H_PF] = ld_frag(zb + a);
      }
      acc_p = mfma32x32x16(wp[ks], uf[ks % K3H_PF], acc_p);
      acc_g = mfma32x32x16(wg[ks], zf[ks % K3H_PF], acc_g);
      at_kstep(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      float o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = sigmoid_f(acc_g[4 * rg + q]) * acc_p[4 * rg + q];
      const u32x2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      *reinterpret_cast<u32x2*>(sm.o[b] + ooff<C>(l32, 2 * (4 * nb + rg) + lhi)) = packed;
    }
  };

  const int sub = lane & 7;                 // sub-lane of a LayerNorm pair (stage-1 mapping)
  if (wave < 4) {
    // ---- waves 0-3: y of channels 64 w .. 64 w + 63, LayerNorm_out of pairs 8 w .. 8 w + 7 ----
    const int w = wave;
    // y of a whole 64-pair tile goes to ys once, as full 128-byte lines of
    // the y planes. LDS row R (128 bytes) holds channel R ^ ((R >> 1) & 1),
    // its 16-byte chunk c (8 pairs) at position c ^ (4 ((R >> 2) & 1)), so
    // that the transpose reads of either half tile are conflict-free. Load q
    // of this wave fills rows 64 w + 8 q .. + 7 (channels of its own slice):
    // lane l gets row 64 w + 8 q + l / 8 at position l % 8, one lane offset
    // plus a uniform 8 channels per load.
    const size_t ch_stride = size_t(p.B) * N * p.n_pad;
    const int yrow = lane >> 3;
    const int ych = yrow ^ ((yrow >> 1) & 1);
    const int yc = (lane & 7) ^ (4 * ((yrow >> 2) & 1));
    const uint32_t yoff = (uint32_t(64 * w + ych) * uint32_t(ch_stride) + 8u * uint32_t(yc)) * 2u;
    const uint32_t cs2 = uint32_t(ch_stride) * 2u;
    auto y_base = [&](int t) {               // the block's 64-pair tile t
      int row, j0;
      half_at(2 * t, row, j0);
      return reinterpret_cast<const char*>(p.plane_y + size_t(row) * p.n_pad + j0);
    };
    auto load_y = [&](const char* base, int q) {
      load_lds16_asm(base + 8u * uint32_t(q) * cs2, yoff, sm.ys + (NLY * w + q) * 1024);
    };
    // Transpose of half tile `half` of ys: item it of lane l is channel pair
    // cp = 32 w + 16 it + l / 4 (channels 2 cp, 2 cp + 1) at pairs 8 jc ..
    // 8 jc + 7 of the half, jc = l % 4. Both layouts are XOR swizzles, so
    // every address is one of a few lane values XOR-ed with a constant plus a
    // constant offset: the read of channel 2 cp + e is yrd[e] ^ 64 half, + 4 KB
    // for item 1; pair 8 jc + 2 q + e of item it goes to u row bytes
    // (uwr ^ 64 it ^ 16 e ^ 128 (q % 2)) + 512 (2 q + e).
    const int jc = lane & 3, cpl = lane >> 2;
    int yrd[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ch = 2 * (32 * w + cpl) + e;
      const int r = ch ^ ((ch >> 1) & 1);
      yrd[e] = r * 128 + jc * 16 + 64 * ((r >> 2) & 1);
    }
    const int uwr = jc * 4096 + (((8 * w + (cpl >> 2)) ^ swz32(8 * jc)) << 4) + 4 * (cpl & 3);
    u32x4 ya, yb;
    auto tr_read = [&](int half, int it) {
      ya = ld16(sm.ys + (yrd[0] ^ (64 * half)) + 4096 * it);
      yb = ld16(sm.ys + (yrd[1] ^ (64 * half)) + 4096 * it);
    };
    // part j of 2 of item it: pairs 8 jc + 4 j .. + 3
    auto tr_write = [&](int b, int it, int j) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = 2 * j + qq;
        const uint32_t even = __builtin_amdgcn_perm(yb[q], ya[q], 0x05040100u);   // pair 8jc + 2q
        const uint32_t odd = __builtin_amdgcn_perm(yb[q], ya[q], 0x07060302u);    // pair 8jc + 2q + 1
        const int a = uwr ^ (64 * it) ^ (128 * (q & 1));
        *reinterpret_cast<uint32_t*>(sm.u[b] + a + 512 * (2 * q)) = even;
        *reinterpret_cast<uint32_t*>(sm.u[b] + (a ^ 16) + 512 * (2 * q + 1)) = odd;
      }
    };
    auto transpose = [&](int b, int half) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        tr_read(half, it);
        tr_write(b, it, 0);
        tr_write(b, it, 1);
      }
    };
    // the transpose spread over the first k-steps of the MFMAs
    auto tr_at = [&](int ks, int b, int half) {
      if (ks == 0) tr_read(half, 0);
      if (ks == 2) tr_write(b, 0, 0);
      if (ks == 3) tr_write(b, 0, 1);
      if (ks == 3) tr_read(half, 1);
      if (ks == 5) tr_write(b, 1, 0);
      if (ks == 6) tr_write(b, 1, 1);
    };
    const uint32_t xo_bytes = uint32_t(p.B) * uint32_t(N) * uint32_t(N) * uint32_t(CZ) * 2u;
    const auto rsrc_o = __builtin_amdgcn_make_buffer_rsrc(p.out, 0, xo_bytes, 0x00020000);
    // pair-major stores of half tile h from o[h % 2]; a pair past N, or a
    // half tile outside the block's, goes past the end of out (0x80000000
    // plus a tile base below 2^31 stays below 2^32) and is dropped
    auto store = [&](int h) {
      const bool valid = h >= 0 && h < nh;
      int row, j0;
      half_at(valid ? h : 0, row, j0);
      const int so = __builtin_amdgcn_readfirstlane((row * N + j0) * CZ * 2);
      const uint8_t* ob = sm.o[h & 1];
#pragma unroll
      for (int it = 0; it < NST; ++it) {
        const int id = it * 256 + tid;
        const int pr = id / (CZ / 8);
        const int cc = id - pr * (CZ / 8);
        u32x4 v = ld16(ob + pr * 512 + ((cc ^ ((pr & 31) >> 1)) << 4));
        if (pr & 1) v = u32x4{v[2], v[3], v[0], v[1]};
        const uint32_t off = (valid && j0 + pr < N) ? uint32_t(id) * 16u : 0x80000000u;
        buffer_store16(rsrc_o, v, off + uint32_t(so));
      }
    };
    const int lp = 8 * w + (lane >> 3);
    auto ln_out = [&](int b) {
      u32x4 yr[NV], u[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) yr[v] = ld16(sm.u[b] + soff32(lp, sub + 8 * v));
      layer_norm_row_lds<NV>(yr, sm.outw, sm.outb, sub, p.eps, u);
#pragma unroll
      for (int v = 0; v < NV; ++v) st16(sm.u[b] + soff32(lp, sub + 8 * v), u[v]);
    };

    {
      const char* base = y_base(0);
#pragma unroll
      for (int q = 0; q < NLY; ++q) load_y(base, q);
    }
    lds_barrier();                           // the staged affines
    wait_vm<0>();
    transpose(0, 0);
    lds_barrier();                           // y rows of half tile 0 (z of half tile 0)
    ln_out(0);
    lds_barrier();                           // u of half tile 0
    for (int h = 0; h < nh; ++h) {
      const int b = h & 1;
      // Half tile h + 1 is the second half of the tile in ys, or the first
      // half of the next tile, whose loads went out one iteration ago
      // (followed by that iteration's stores). Its transpose runs between
      // the MFMAs of the first k-steps; once both halves of tile h / 2 have
      // been read out of ys, the next tile's y goes in, one load per k-step,
      // so that the issue waits overlap the MFMAs.
      if (h + 1 < nh) {
        if ((h & 1) == 1) wait_vm<NST>();
        const int bn = b ^ 1, half = (h + 1) & 1;
        if ((h & 1) == 0 && (h >> 1) + 1 < nk) {
          const char* base = y_base((h >> 1) + 1);
          mma_gate(b, [&](int ks) {
            tr_at(ks, bn, half);
            if (ks == 7) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (ks >= 8) load_y(base, ks - 8);
          });
        } else {
          mma_gate(b, [&](int ks) { tr_at(ks, bn, half); });
        }
      } else {
        mma_gate(b, [](int) {});
      }
      lds_barrier();
      if (h + 1 < nh) ln_out(b ^ 1);
      store(h - 1);
      lds_barrier();
    }
    store(nh - 1);
  } else {
    // ---- waves 4-7: x and LayerNorm_in of pairs 8 lw .. 8 lw + 7 ----
    const int lw = wave - 4;
    // x of a half tile -> xs, 512 bytes per pair row, 16-byte chunk c of pair
    // lp at position c ^ (8 (lp & 1)); a pair past N reads pair N - 1 (its
    // results are not stored). Load q of this wave fills rows 8 lw + 2 q,
    // 8 lw + 2 q + 1: the rows its LayerNorm lanes read.
    auto load_x = [&](int h) {
      int row, j0;
      half_at(min(h, nh - 1), row, j0);
      const char* base = reinterpret_cast<const char*>(p.x + size_t(row) * N * CZ);
#pragma unroll
      for (int q = 0; q < NLD; ++q) {
        const int s = (NLD * lw + q) * 64 + lane;
        const int pr = s >> 5, pos = s & 31;
        const int c = pos ^ ((pr & 1) << 3);
        const uint32_t off = (uint32_t(min(j0 + pr, N - 1)) * CZ + 8u * uint32_t(c)) * 2u;
        load_lds16_asm(base, off, sm.xs + (NLD * lw + q) * 1024);
      }
    };
    const int lp = 8 * lw + (lane >> 3);
    // LayerNorm_in of the x in xs into z[b]; once the row is in registers,
    // xs takes the next loads (`then`)
    auto ln_in = [&](int b, auto&& then) {
      u32x4 xr[NV], z[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) xr[v] = ld16(sm.xs + lp * 512 + (((sub + 8 * v) ^ ((lp & 1) << 3)) << 4));
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      then();
      layer_norm_row_lds<NV>(xr, sm.inw, sm.inb, sub, p.eps, z);
#pragma unroll
      for (int v = 0; v < NV; ++v) st16(sm.z[b] + soff32(lp, sub + 8 * v), z[v]);
    };
    load_x(0);
    lds_barrier();                           // the staged affines
    wait_vm<0>();
    ln_in(0, [&] { load_x(1); });
    lds_barrier();                           // z of half tile 0 (y rows of half tile 0)
    lds_barrier();                           // u of half tile 0
    for (int h = 0; h < nh; ++h) {
      const int b = h & 1;
      if (h + 1 < nh) {
        wait_vm<0>();                        // x of half tile h + 1 (all this wave has in flight)
        ln_in(b ^ 1, [&] {
          if (h + 2 < nh) load_x(h + 2);
        });
      }
      lds_barrier();
      mma_gate(b, [](int) {});
      lds_barrier();
    }
  }
  // every direct load has been waited for above; nothing may still be
  // writing the LDS when the block ends
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
//   phase 1: matrix waves run tile k's MFMAs (u/z buffer k % 2); LayerNorm
//            waves write z of tile k+1
//   phase 2: matrix waves run both pair halves' gates, transpose the y of
//            tile k+2 (in registers) into y rows k % 2, store tile k-1 and
//            load y of tile k+4; LayerNorm waves write u of tile k+1 from y
//            rows (k+1) % 2.
// With two sets of y rows the transpose runs a tile ahead, in the phase the
// LayerNorm waves' LayerNorm_out makes the longer one. The LayerNorm waves
// load x of tile k+3 in phase 1, right after their LayerNorm_in has read the
// register set the loads go to (two register sets each: x and y have 2
// iterations to land); phase 2 then holds the matrix waves' y loads and
// stores alone.
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
  uint8_t y[2][K3_TP * RB];                // transposed y rows of the next two tiles
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
          *reinterpret_cast<uint32_t*>(sm.y[e] + soff<C>(r0, cp >> 2) + 4 * (cp & 3)) = even;
          *reinterpret_cast<uint32_t*>(sm.y[e] + soff<C>(r0 + 1, cp >> 2) + 4 * (cp & 3)) = odd;
        }
      }
    };
    // prologue: the y rows of tiles 0 and 1, with y of tiles 2 and 3 in
    // flight, each into the register set its tile's transpose has just read
    // (the stores of a first iteration go past the end of out)
    prefetch_y(0, I0{});
    prefetch_y(1, I1{});
    store(-2);
    transpose(I0{});
    prefetch_y(2, I0{});
    transpose(I1{});
    prefetch_y(3, I1{});
    lds_barrier();                           // y rows of tiles 0, 1 (the LayerNorm waves: z of tile 0)
    lds_barrier();                           // u of tile 0
    // iteration k: tile k's matrix work; the y of tile k + 2 (set k % 2)
    // transposed, then refilled with tile k + 4
    auto iteration = [&](int k, auto set) {
      const int b = k & 1;
      f32x16 p0, g0, p1, g1;
      if (k < nk) {
        mma(b, 0, p0, g0);
        mma(b, 1, p1, g1);
      }
      lds_barrier();
      if (k < nk) {
        gate(b, 0, p0, g0);
        gate(b, 1, p1, g1);
      }
      if (k + 2 < nk) transpose(set);
      store(k - 1);
      prefetch_y(k + 4, set);
      lds_barrier();
    };
    for (int k = 0; k < nit; k += 2) {
      iteration(k, I0{});
      iteration(k + 1, I1{});
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
        y0[v] = ld16(sm.y[b] + soff<C>(P0, sub + 8 * v));
        y1[v] = ld16(sm.y[b] + soff<C>(P1, sub + 8 * v));
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
    hipLaunchKernelGGL(k3_epilogue_h256, dim3(grid_x), dim3(K3_THREADS), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace trimul
