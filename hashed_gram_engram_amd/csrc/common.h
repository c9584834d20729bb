// Device helpers shared by the Engram kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace engram {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kFltMax = 3.40282347e38f;

// ------------------------------------------------------------------ bf16 packing

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 p = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_round(float v) {
  return bf16_lo(pack_bf16x2(v, 0.0f));
}

// Any NaN half of a packed bf16 pair becomes the canonical quiet NaN 0x7FC0 (the hardware
// convert keeps the NaN's sign; the table dequantisation contract writes 0x7FC0).
__device__ __forceinline__ uint32_t canon_nan2(uint32_t w) {
  uint32_t lo = w & 0xFFFFu, hi = w >> 16;
  lo = ((lo & 0x7FFFu) > 0x7F80u) ? 0x7FC0u : lo;
  hi = ((hi & 0x7FFFu) > 0x7F80u) ? 0x7FC0u : hi;
  return lo | (hi << 16);
}

// ------------------------------------------------------------------ fp8 dequantisation

// Non-zero iff one of the four e4m3fn codes in `c` is a NaN code (low seven bits all ones).
__device__ __forceinline__ uint32_t nan_code_bits(uint32_t c) {
  return ((c & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
}

// E8M0 block scale (OCP MX v1.0, the scale of the MXFP8 tables): 2^(e - 127) for e = 0..254,
// NaN for 255.  e = 0 is the fp32 subnormal 2^-127; every other value is a normal fp32 whose
// exponent field is e.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  const uint32_t bits = e == 0u ? 0x00400000u : (e == 255u ? 0x7FC00000u : e << 23);
  return __uint_as_float(bits);
}

// Scale idx of a table's block scales: fp32, or E8M0 bytes.
__device__ __forceinline__ float load_scale(const void* scales, int64_t idx, int e8m0) {
  return e8m0 ? e8m0_to_f32(static_cast<const uint8_t*>(scales)[idx]) : static_cast<const float*>(scales)[idx];
}

// Four codes times one fp32 scale -> four bf16 in two dwords.  The fp8 decode is exact
// (v_cvt_pk_f32_fp8, OCP e4m3), the product is one IEEE fp32 multiply and the bf16 rounding is
// nearest-even; NaN results are not canonicalised here.
__device__ __forceinline__ u32x2 dequant4_raw(uint32_t c, float s) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(c, true);
  u32x2 r;
  r.x = pack_bf16x2(lo.x * s, lo.y * s);
  r.y = pack_bf16x2(hi.x * s, hi.y * s);
  return r;
}

// Sixteen codes with one scale -> sixteen bf16 (o0 = features 0..7, o1 = 8..15).  A NaN result
// can only come from a NaN code or a non-finite scale; both are rare, so the canonicalisation
// runs behind a branch that the whole wave normally skips.
__device__ __forceinline__ void dequant16(u32x4 c, float s, u32x4& o0, u32x4& o1) {
  u32x2 a = dequant4_raw(c.x, s), b = dequant4_raw(c.y, s);
  u32x2 d = dequant4_raw(c.z, s), e = dequant4_raw(c.w, s);
  o0 = u32x4{a.x, a.y, b.x, b.y};
  o1 = u32x4{d.x, d.y, e.x, e.y};
  uint32_t bad = nan_code_bits(c.x) | nan_code_bits(c.y) | nan_code_bits(c.z) | nan_code_bits(c.w);
  if (__builtin_expect(bad != 0u || !(__builtin_fabsf(s) <= kFltMax), 0)) {
    o0 = u32x4{canon_nan2(o0.x), canon_nan2(o0.y), canon_nan2(o0.z), canon_nan2(o0.w)};
    o1 = u32x4{canon_nan2(o1.x), canon_nan2(o1.y), canon_nan2(o1.z), canon_nan2(o1.w)};
  }
}

// ------------------------------------------------------------------ MFMA

// D = A * B + C for a 16x16 output block, K = 32 (v_mfma_f32_16x16x32_bf16).  Lane l supplies
// A[l % 16][8 * (l / 16) + e] and B[8 * (l / 16) + e][l % 16], e = 0..7, and receives
// D[4 * (l / 16) + r][l % 16], r = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D = A * B + C for a 16x16 output block, K = 128, A and B fp8 e4m3 codes with one E8M0 scale
// per 32 values (v_mfma_scale_f32_16x16x128_f8f6f4).  Lane l supplies row / column l % 16 of
// A / B: bytes 0..15 at K = 16 (l / 16) + [0, 16), bytes 16..31 at K = 64 + 16 (l / 16) + [0, 16),
// and the scale of K block l / 16 (K [32 (l / 16), 32 (l / 16) + 32)) of that row / column in the
// low byte of sa / sb.  (Layout checked on the device against a host evaluation.)
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
// The two 16-byte parts of a lane's operand as one 8-register tuple.
__device__ __forceinline__ i32x8 mx_operand(u32x4 lo, u32x4 hi) {
  return __builtin_shufflevector(__builtin_bit_cast(i32x4, lo), __builtin_bit_cast(i32x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 mfma_mx16x16x128(i32x8 a, int sa, i32x8 b, int sb, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ f32x4 mfma_mx16x16x128(u32x4 a_lo, u32x4 a_hi, int sa, u32x4 b_lo, u32x4 b_hi, int sb,
                                                  f32x4 c) {
  return mfma_mx16x16x128(mx_operand(a_lo, a_hi), sa, mx_operand(b_lo, b_hi), sb, c);
}

// ------------------------------------------------------------------ reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ------------------------------------------------------------------ cross-workgroup signalling

__device__ __forceinline__ uint32_t atomic_add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_relaxed(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-coherent relaxed accesses (agent scope).  Each one reaches the device coherence point
// instead of a possibly stale per-XCD L2 copy, so small blocks of data handed from one
// workgroup to another need no cache-wide writeback or invalidate (which agent-scope fences
// perform and which cost tens of microseconds per kernel).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same for 16-byte records at byte offset `off` from a wave-uniform base (one
// buffer_store / buffer_load_dwordx4 with the agent-coherent cache policy, sc1): one memory
// transaction per lane instead of four.  Readers only read records whose writers have
// finished (ordered by a counter), so the 16 bytes need no atomicity.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(0x7FFFFFFF), 0x00020000);
}
constexpr int kCpolSc1 = 16;  // cache policy bit: coherent at agent scope
__device__ __forceinline__ void store_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCpolSc1);
}
__device__ __forceinline__ f32x4 load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1));
}

// Waits until every memory operation this wave has issued is complete (stores acknowledged by
// their destination).  Followed by a workgroup barrier, it orders all coherent stores of the
// workgroup before any access that one thread issues after the barrier.
__device__ __forceinline__ void drain_memory_ops() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// Spin (with sleeps) until *p >= target or the spin budget is spent; returns false on time-out.
// Every wait in these kernels is bounded so that a grid always drains.
__device__ __forceinline__ bool wait_at_least(const uint32_t* p, uint32_t target, uint32_t budget) {
  uint32_t it = 0;
  while (load_relaxed(p) < target) {
    __builtin_amdgcn_s_sleep(8);
    if (++it > budget) return false;
  }
  return true;
}

}  // namespace engram
