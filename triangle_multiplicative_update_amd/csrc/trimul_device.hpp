// Device helpers shared by the three gfx950 kernels of the triangle
// multiplicative update: bf16 packing, wave64 cross-lane sums, the two-pass
// LayerNorm of one pair row, the logistic gate, and MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trimul {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 -----

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Two floats -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), lo first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight values of a 16-byte chunk, in memory order.
__device__ __forceinline__ void unpack8(const u32x4& c, float (&v)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = bf16_lo(c[q]);
    v[2 * q + 1] = bf16_hi(c[q]);
  }
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// 16-byte buffer load at byte offset voff + soff (soff uniform)
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// 16-byte buffer store at byte offset voff. The whole offset goes in the
// vector operand and the scalar offset is the constant 0: a store of more
// than 8 bytes reads its data registers over more than one cycle, and the
// compiler only keeps the next instruction from overwriting them when the
// scalar offset is not a register (with a register there, the first data
// dword has been seen to take the value written by the next instruction).
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, const u32x4& v, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}
// 8-byte buffer store at byte offset voff (8 bytes are read in one cycle, so
// the data registers are free for the next instruction)
__device__ __forceinline__ void buffer_store8(__amdgpu_buffer_rsrc_t r, const u32x2& v, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, 0, 0);
}
__device__ __forceinline__ bf16x8 ld_frag(const void* p) { return *reinterpret_cast<const bf16x8*>(p); }

typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte-per-lane global -> LDS copy (direct load, no registers): lane
// l's 16 bytes land at lds + 16 l; `lds` must be the same for the whole wave.
// It counts as a vector-memory operation: wait_vm before reading the bytes.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// The same copy issued as inline assembly, from a uniform base `gbase` plus
// a per-lane 32-bit byte offset. The compiler's wait-count model treats a
// direct load like a flat access that may retire out of order, and while one
// is in flight it waits for zero outstanding operations before every LDS
// read and every use of a loaded register; issued this way the copy is
// invisible to that model, so the compiler's own waits stay exact (an extra
// operation in the counters only makes them wait longer). The caller waits
// for the copy itself with wait_vm. Only for kernels in which no other code
// uses M0 (the LDS address register of the copy).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16_asm(const void* gbase, uint32_t voff, const void* lds) {
  const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// wait until at most n vector-memory operations of this wave are outstanding
// (they retire in issue order)
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// One bf16 from global memory. The address-space cast makes it a global load:
// a flat load also counts against the LDS wait counter, so every later LDS
// wait or barrier would wait for it too.
__device__ __forceinline__ uint16_t ld_global_u16(const uint16_t* p) {
  return *(const __attribute__((address_space(1))) uint16_t*)(p);
}

// bf16 bits -> float, as an instruction the compiler cannot fold back to the
// load that produced them (the shift discards whatever the register's upper
// half holds). A prefetched value converted by plain code is turned into a
// conversion right after its load, and the wait for that load then lands in
// the middle of the work meant to hide it.
__device__ __forceinline__ float bf16_bits_late(uint16_t h) {
  float r;
  asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(r) : "v"(h));
  return r;
}

// ------------------------------------------------------- block barrier ----
// A workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, then meets the other waves. __syncthreads() would also drain
// every outstanding global load and store (s_waitcnt vmcnt(0)), serializing
// the memory traffic of a tile with the compute of the next. The "memory"
// clobber keeps the compiler from moving LDS accesses across it; global
// memory is never used to communicate between waves of a block.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ------------------------------------------------------- cross-lane sums ---

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, false));
}

// Sum over each aligned group of 8 lanes. Every lane of the group ends with the
// same bits: each step adds a lane's value to its partner's, and the two
// partners add the same two numbers.
__device__ __forceinline__ float sum_lanes8(float v) {
  v = v + dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]: partner lane ^ 1
  v = v + dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]: partner lane ^ 2
  v = v + dpp_f<0x141>(v);  // row_half_mirror: lane i <-> 7 - i inside 8 lanes
  return v;
}

// ------------------------------------------------------- LDS swizzle ----
//
// LDS bank model of gfx950, measured (per-instruction throughput of
// ds_read/ds_write patterns at 8 waves per CU): 64 banks of 4 bytes (one
// 256-byte line per cycle). A 16-byte access runs in 4 cycles of 16 lanes,
// the cycle of lane l being (bit 5 of l, parity of bits 2..4 of l): lanes
// 0-3, 12-15, 20-23, 24-27 share one cycle, 4-7, 8-11, 16-19, 28-31 the next,
// and likewise in the upper half. An 8-byte access runs in 2 cycles of 32
// lanes, the cycle being the parity of lane bits 5 and 1. Within a cycle the
// lanes must hit distinct banks (identical addresses excepted).
//
// Pair-major tiles with 256-byte rows (128 bf16 channels) place 16-byte slot
// `s` of row `r` at slot s ^ lds_swz(r), with the row bits XOR-ed in as
// bit 0 -> 1, bit 1 -> 8, bit 3 -> 2, bit 4 -> 4, bit 5 -> 8 (bit 2 -> 0). Under
// the model this keeps every access of the stage-3 tiles conflict-free: the
// MFMA fragment reads (32 consecutive rows at one slot, the upper half at the
// next slot), the LayerNorm rows (8 lanes x 16 bytes per row, 8 rows), and the
// transposing 4-byte writes of 8 rows {8j + e} x 8 consecutive dwords (found
// by exhaustive search over such linear swizzles, checked on the GPU).
__device__ __forceinline__ int lds_swz(int r) {
  return ((r & 1) ? 1 : 0) ^ ((r & 2) ? 8 : 0) ^ ((r & 8) ? 2 : 0) ^ ((r & 16) ? 4 : 0) ^ ((r & 32) ? 8 : 0);
}

// ------------------------------------------------------------ LayerNorm ----
//
// One pair row of length 64*NV is held by 8 consecutive lanes; lane `sub`
// holds the NV chunks starting at element 8*sub + 64*v. Statistics in fp32,
// two passes (mean, then mean of squared deviations, biased), eps inside the
// square root, affine after normalisation, result rounded once to bf16. The
// summation order is fixed (partial sums, then the 8-lane reduction). The
// stage-1 and stage-3 kernels both call this with the same lane mapping, so
// stage 3's recomputed z_in has the bits stage 1 used.
// Rows of 4 or more chunks per lane (c_z = 256) unpack the bf16 input again
// in each pass instead of keeping 8 * NV floats live across the two
// reductions; the values, and so the result bits, are the same either way.
// Those rows go through the three passes below, which a kernel may also call
// one at a time (with the row re-read in between): the same operations in the
// same order, so the same bits.

// The passes are also available one 16-byte chunk at a time (c = 0, 1, ...
// in order), for kernels that spread a row's LayerNorm over other work.
// pass 1: partial sums of chunk c (element i = 8 c + e into sum i % 4)
__device__ __forceinline__ void ln_sum_chunk(float (&sp)[4], const u32x4& x, int c) {
#pragma clang fp contract(off)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = 8 * c + e;
    const float v = (e & 1) ? bf16_hi(x[e >> 1]) : bf16_lo(x[e >> 1]);
    sp[i & 3] = (i < 4) ? v : sp[i & 3] + v;
  }
}
// the row mean from the partial sums (every lane of the 8 ends with the same bits)
template <int NV>
__device__ __forceinline__ float ln_mean_of(const float (&sp)[4]) {
#pragma clang fp contract(off)
  constexpr float inv_n = 1.0f / float(64 * NV);
  return sum_lanes8((sp[0] + sp[1]) + (sp[2] + sp[3])) * inv_n;
}
// pass 2: partial sums of squared deviations of chunk c
__device__ __forceinline__ void ln_sq_chunk(float (&ssp)[4], const u32x4& x, int c, float mean) {
#pragma clang fp contract(off)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = 8 * c + e;
    const float d = ((e & 1) ? bf16_hi(x[e >> 1]) : bf16_lo(x[e >> 1])) - mean;
    ssp[i & 3] = (i < 4) ? d * d : __builtin_fmaf(d, d, ssp[i & 3]);
  }
}
// 1 / sqrt(biased variance + eps) from the partial sums
template <int NV>
__device__ __forceinline__ float ln_rstd_of(const float (&ssp)[4], float eps) {
#pragma clang fp contract(off)
  constexpr float inv_n = 1.0f / float(64 * NV);
  const float var = sum_lanes8((ssp[0] + ssp[1]) + (ssp[2] + ssp[3])) * inv_n;
  return __builtin_amdgcn_rsqf(var + eps);
}
// pass 3 on one chunk: normalise, affine, round to bf16
__device__ __forceinline__ u32x4 ln_apply_chunk(const u32x4& x, float mean, float rstd, const float (&wv)[8],
                                                const float (&bv)[8]) {
#pragma clang fp contract(off)
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = (e & 1) ? bf16_hi(x[e >> 1]) : bf16_lo(x[e >> 1]);
    o[e] = __builtin_fmaf((v - mean) * rstd, wv[e], bv[e]);
  }
  return u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
}

// the three passes over a whole row held by the lane
template <int NV>
__device__ __forceinline__ float ln_mean(const u32x4 (&x)[NV]) {
  float sp[4];
#pragma unroll
  for (int c = 0; c < NV; ++c) ln_sum_chunk(sp, x[c], c);
  return ln_mean_of<NV>(sp);
}
template <int NV>
__device__ __forceinline__ float ln_rstd(const u32x4 (&x)[NV], float mean, float eps) {
  float ssp[4];
#pragma unroll
  for (int c = 0; c < NV; ++c) ln_sq_chunk(ssp, x[c], c, mean);
  return ln_rstd_of<NV>(ssp, eps);
}
template <int NV, class WB>
__device__ __forceinline__ void ln_apply(const u32x4 (&x)[NV], float mean, float rstd, WB&& affine,
                                         u32x4 (&z)[NV]) {
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    float wv[8], bv[8];
    affine(c, wv, bv);
    z[c] = ln_apply_chunk(x[c], mean, rstd, wv, bv);
  }
}

template <int NV, class WB>
__device__ __forceinline__ void layer_norm_row_wb(const u32x4 (&xin)[NV], WB&& affine, float eps,
                                                  u32x4 (&zout)[NV]) {
#pragma clang fp contract(off)
  if constexpr (NV > 2) {
    const float mean = ln_mean<NV>(xin);
    ln_apply<NV>(xin, mean, ln_rstd<NV>(xin, mean, eps), affine, zout);
  } else {
    constexpr float inv_n = 1.0f / float(64 * NV);
    float v[NV][8];
#pragma unroll
    for (int c = 0; c < NV; ++c) unpack8(xin[c], v[c]);
    // in-lane sums as four interleaved partial sums (element i into sum i % 4),
    // combined pairwise: dependency chains of 4 + 2 instead of 16, which a
    // single wave per SIMD can issue without stalling
    float sp[4];
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * c + e;
        sp[i & 3] = (i < 4) ? v[c][e] : sp[i & 3] + v[c][e];
      }
    float s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
    s = sum_lanes8(s);
    const float mean = s * inv_n;
    float ssp[4];
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * c + e;
        const float d = v[c][e] - mean;
        ssp[i & 3] = (i < 4) ? d * d : __builtin_fmaf(d, d, ssp[i & 3]);
      }
    float ss = (ssp[0] + ssp[1]) + (ssp[2] + ssp[3]);
    ss = sum_lanes8(ss);
    const float var = ss * inv_n;
    const float rstd = __builtin_amdgcn_rsqf(var + eps);
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      float wv[8], bv[8];
      affine(c, wv, bv);
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf((v[c][e] - mean) * rstd, wv[e], bv[e]);
      zout[c] = u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                      pack_bf16x2(o[6], o[7])};
    }
  }
}

// R rows at once: every step is taken for each row before the next step, so
// the rows' dependency chains (the lane reductions above all) overlap where
// one wave per SIMD would otherwise wait on each. affine(r, c, wv, bv) gives
// row r's affine for chunk c. Each row sees exactly the operations of
// layer_norm_row_wb in the same order, so its bits are the same (rows of 4 or
// more chunks per lane are re-unpacked per pass, as there).
template <int NV, int R, class WB>
__device__ __forceinline__ void layer_norm_rows_wb(const u32x4 (&x)[R][NV], WB&& affine, float eps,
                                                   u32x4 (&z)[R][NV]) {
#pragma clang fp contract(off)
  constexpr float inv_n = 1.0f / float(64 * NV);
  constexpr bool kKeep = NV <= 2;
  float v[R][kKeep ? NV : 1][8];
  auto elem = [&](int r, int c, int e) -> float {
    if constexpr (kKeep) return v[r][c][e];
    else return (e & 1) ? bf16_hi(x[r][c][e >> 1]) : bf16_lo(x[r][c][e >> 1]);
  };
  if constexpr (kKeep) {
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int r = 0; r < R; ++r) unpack8(x[r][c], v[r][c]);
  }
  float sp[R][4];
#pragma unroll
  for (int c = 0; c < NV; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 8 * c + e;
#pragma unroll
      for (int r = 0; r < R; ++r) sp[r][i & 3] = (i < 4) ? elem(r, c, e) : sp[r][i & 3] + elem(r, c, e);
    }
  float s[R], mean[R];
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = (sp[r][0] + sp[r][1]) + (sp[r][2] + sp[r][3]);
  // sum_lanes8 on every row, step by step
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = s[r] + dpp_f<0xB1>(s[r]);
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = s[r] + dpp_f<0x4E>(s[r]);
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = s[r] + dpp_f<0x141>(s[r]);
#pragma unroll
  for (int r = 0; r < R; ++r) mean[r] = s[r] * inv_n;
  float ssp[R][4];
#pragma unroll
  for (int c = 0; c < NV; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 8 * c + e;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float d = elem(r, c, e) - mean[r];
        ssp[r][i & 3] = (i < 4) ? d * d : __builtin_fmaf(d, d, ssp[r][i & 3]);
      }
    }
  float ss[R], rstd[R];
#pragma unroll
  for (int r = 0; r < R; ++r) ss[r] = (ssp[r][0] + ssp[r][1]) + (ssp[r][2] + ssp[r][3]);
#pragma unroll
  for (int r = 0; r < R; ++r) ss[r] = ss[r] + dpp_f<0xB1>(ss[r]);
#pragma unroll
  for (int r = 0; r < R; ++r) ss[r] = ss[r] + dpp_f<0x4E>(ss[r]);
#pragma unroll
  for (int r = 0; r < R; ++r) ss[r] = ss[r] + dpp_f<0x141>(ss[r]);
#pragma unroll
  for (int r = 0; r < R; ++r) rstd[r] = __builtin_amdgcn_rsqf(ss[r] * inv_n + eps);
#pragma unroll
  for (int c = 0; c < NV; ++c) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float wv[8], bv[8], o[8];
      affine(r, c, wv, bv);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf((elem(r, c, e) - mean[r]) * rstd[r], wv[e], bv[e]);
      z[r][c] = u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                      pack_bf16x2(o[6], o[7])};
    }
  }
}

// two rows with one affine held in registers as packed bf16
template <int NV>
__device__ __forceinline__ void layer_norm_rows2(const u32x4 (&x0)[NV], const u32x4 (&x1)[NV],
                                                 const u32x4 (&w)[NV], const u32x4 (&b)[NV], float eps,
                                                 u32x4 (&z0)[NV], u32x4 (&z1)[NV]) {
  u32x4 x[2][NV], z[2][NV];
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    x[0][c] = x0[c];
    x[1][c] = x1[c];
  }
  layer_norm_rows_wb<NV, 2>(x, [&](int, int c, float (&wv)[8], float (&bv)[8]) {
    unpack8(w[c], wv);
    unpack8(b[c], bv);
  }, eps, z);
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    z0[c] = z[0][c];
    z1[c] = z[1][c];
  }
}

// fp32 affine rows in LDS (see layer_norm_row_lds): this lane's 8 + 8 values of chunk c
__device__ __forceinline__ void lds_affine8(const float* w, const float* b, int sub, int c, float (&wv)[8],
                                            float (&bv)[8]) {
  const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + 8 * sub + 64 * c);
  const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + 8 * sub + 64 * c + 4);
  const f32x4 b0 = *reinterpret_cast<const f32x4*>(b + 8 * sub + 64 * c);
  const f32x4 b1 = *reinterpret_cast<const f32x4*>(b + 8 * sub + 64 * c + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    wv[e] = w0[e];
    wv[4 + e] = w1[e];
    bv[e] = b0[e];
    bv[4 + e] = b1[e];
  }
}

// affine parameters held in registers as packed bf16 (chunk c of this lane)
template <int NV>
__device__ __forceinline__ void layer_norm_row(const u32x4 (&xin)[NV], const u32x4 (&w)[NV],
                                               const u32x4 (&b)[NV], float eps, u32x4 (&zout)[NV]) {
  layer_norm_row_wb<NV>(xin, [&](int c, float (&wv)[8], float (&bv)[8]) {
    unpack8(w[c], wv);
    unpack8(b[c], bv);
  }, eps, zout);
}

// affine parameters as fp32 arrays in LDS (the full row; this lane reads the
// 8 + 8 values of each of its chunks, the same for every pair): the same
// arithmetic as the register form, for kernels without registers to spare
template <int NV>
__device__ __forceinline__ void layer_norm_row_lds(const u32x4 (&xin)[NV], const float* w, const float* b,
                                                   int sub, float eps, u32x4 (&zout)[NV]) {
  layer_norm_row_wb<NV>(xin, [&](int c, float (&wv)[8], float (&bv)[8]) { lds_affine8(w, b, sub, c, wv, bv); },
                        eps, zout);
}

// Widen a bf16 vector of length n into an fp32 LDS array (block-cooperative;
// the caller synchronises before the first read). A NULL source gives zeros.
__device__ __forceinline__ void stage_f32(float* dst, const uint16_t* src, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src ? bf16_to_f32(src[i]) : 0.0f;
}

// ------------------------------------------------------------- sigmoid -----
// 1 / (1 + 2^(-g log2 e)) on the hardware exp2 and reciprocal. Saturates to 0
// and 1 at the extremes (exp2 -> inf gives 1/inf = 0; exp2 -> 0 gives 1).
__device__ __forceinline__ float sigmoid_f(float g) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// sigmoid(g) * v * m with the mask folded into the exponent and denominator:
// v / ((1 + 2^t) * mi) with t = -g log2 e + mb, where (mb, mi) = (+inf, 1)
// for m = 0 and (0, 1/m) otherwise. m = 0 gives 2^inf = inf, 1 / inf = 0 and
// fma(v, 0, +0.0) = +0.0 exactly; m = 1 gives the same bits as
// sigmoid_f(g) * v. The final fma with +0.0 turns a -0.0 product into +0.0.
__device__ __forceinline__ float gate_masked(float g, float v, float mb, float mi) {
  const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(g, -1.4426950408889634f, mb));
  return __builtin_fmaf(v, __builtin_amdgcn_rcpf(__builtin_fmaf(e, mi, mi)), 0.0f);
}

// ---------------------------------------------------------------- MFMA -----

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D (16 x 16) += A (16 x 32) B (32 x 16): lane l supplies row l % 16 of A and
// column l % 16 of B, each at k = 8 (l / 16) .. + 7, and receives
// D[4 (l / 16) + i][l % 16] in register i
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace trimul
