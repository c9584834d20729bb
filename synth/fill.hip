// Device-side fill of seeded synthetic inputs (test and benchmark infrastructure).
//
// Implements exactly the element definitions documented in synth/__init__.py, so that any
// element written here equals the one the host generator produces for the same key and
// index.  Holds none of the Engram method's arithmetic.  Double-precision steps are kept
// unfused (fp contract off) because the host evaluates them as separate IEEE operations.
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * kGolden);
}

// nearest-even e4m3 magnitude code of r * 2^-22, 0 <= r < 2^24
__device__ __forceinline__ uint32_t e4m3_mag(uint32_t r) {
  if (r < (1u << 16)) {  // subnormal grid, quantum 2^13 units
    uint32_t t = r >> 13, rem = r & 0x1FFFu, half = 0x1000u;
    if (rem > half || (rem == half && (t & 1u))) ++t;
    return t;  // t == 8 is the smallest normal code 0x08
  }
  int p = 31 - __clz(r);
  int q = p - 3;
  uint32_t t = r >> q, rem = r & ((1u << q) - 1u), half = 1u << (q - 1);
  if (rem > half || (rem == half && (t & 1u))) ++t;
  int e = p - 15;
  if (t == 16u) { t = 8u; ++e; }
  return (uint32_t(e) << 3) | (t - 8u);
}

__device__ __forceinline__ uint16_t bf16_rne_bits(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return uint16_t(b >> 16);
}

__device__ __forceinline__ float normal_f32(uint64_t key, uint64_t i, double mean, double stdv) {
  int64_t s = 0;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    uint64_t d = draw(key, 3 * i + k);
#pragma unroll
    for (int f = 0; f < 4; ++f) s += int64_t((d >> (16 * f)) & 0xFFFFull);
  }
  double z = double(s + 6 - 393216) / 65536.0;
  double p = stdv * z;
  double v = mean + p;
  return float(v);
}

__global__ void k_fill_codes(uint8_t* __restrict__ dst, int64_t first, int64_t n, uint64_t key) {
  // each thread writes 8 consecutive codes (one 64-bit store when aligned)
  int64_t stride = int64_t(gridDim.x) * blockDim.x * 8;
  for (int64_t i = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 8; i < n; i += stride) {
    uint64_t packed = 0;
    int cnt = (n - i) < 8 ? int(n - i) : 8;
    for (int e = 0; e < cnt; ++e) {
      uint64_t d = draw(key, uint64_t(first + i + e));
      uint32_t code = uint32_t(d >> 63) << 7 | e4m3_mag(uint32_t((d >> 32) & 0xFFFFFFull));
      packed |= uint64_t(code) << (8 * e);
    }
    if (cnt == 8 && ((reinterpret_cast<uintptr_t>(dst + i) & 7) == 0)) {
      *reinterpret_cast<uint64_t*>(dst + i) = packed;
    } else {
      for (int e = 0; e < cnt; ++e) dst[i + e] = uint8_t(packed >> (8 * e));
    }
  }
}

__global__ void k_fill_uniform_f32(float* __restrict__ dst, int64_t first, int64_t n,
                                   uint64_t key, double lo, double hi) {
  int64_t stride = int64_t(gridDim.x) * blockDim.x;
  double w = hi - lo;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    uint64_t d = draw(key, uint64_t(first + i));
    double u = double(d >> 40) * 0x1p-24;
    double p = w * u;
    dst[i] = float(lo + p);
  }
}

// E8M0 exponent bytes, uniform integers in [lo, hi]: lo + ((draw >> 40) * (hi - lo + 1)) >> 24.
__global__ void k_fill_e8m0(uint8_t* __restrict__ dst, int64_t first, int64_t n, uint64_t key,
                            uint32_t lo, uint32_t span) {
  int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    uint64_t d = draw(key, uint64_t(first + i));
    dst[i] = uint8_t(lo + uint32_t(((d >> 40) * uint64_t(span)) >> 24));
  }
}

__global__ void k_fill_normal_bf16(uint16_t* __restrict__ dst, int64_t first, int64_t n,
                                   uint64_t key, double mean, double stdv) {
  int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = bf16_rne_bits(normal_f32(key, uint64_t(first + i), mean, stdv));
}

__global__ void k_fill_x(uint16_t* __restrict__ dst, int64_t tok0, int64_t ntok, int64_t per_tok,
                         uint64_t key_x, uint64_t key_out, uint32_t thr, double stdv,
                         double out_std) {
  int64_t n = ntok * per_tok;
  int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    int64_t tok = tok0 + i / per_tok;
    bool outlier = thr != 0u && uint32_t(draw(key_out, uint64_t(tok)) >> 40) < thr;
    uint64_t gi = uint64_t(tok0 * per_tok + i);
    dst[i] = bf16_rne_bits(normal_f32(key_x, gi, 0.0, outlier ? out_std : stdv));
  }
}

inline unsigned grid_for(int64_t work_items, int threads) {
  int64_t g = (work_items + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return unsigned(g);
}

}  // namespace

extern "C" {

// Fills nrows table rows of head_dim codes starting at row `row0`; dst points at row row0.
int synth_fill_codes(uint8_t* dst, int64_t row0, int64_t nrows, int32_t head_dim, uint64_t key,
                     hipStream_t stream) {
  int64_t n = nrows * head_dim;
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fill_codes, dim3(grid_for((n + 7) / 8, 256)), dim3(256), 0, stream, dst,
                     row0 * head_dim, n, key);
  return int(hipGetLastError());
}

// Fills nrows x n_blocks fp32 scales U(lo, hi); dst points at row row0.
int synth_fill_scales(float* dst, int64_t row0, int64_t nrows, int32_t n_blocks, uint64_t key,
                      double lo, double hi, hipStream_t stream) {
  int64_t n = nrows * n_blocks;
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fill_uniform_f32, dim3(grid_for(n, 256)), dim3(256), 0, stream, dst,
                     row0 * n_blocks, n, key, lo, hi);
  return int(hipGetLastError());
}

// Fills nrows x n_blocks E8M0 scale bytes, uniform in [lo, hi]; dst points at row row0.
int synth_fill_e8m0(uint8_t* dst, int64_t row0, int64_t nrows, int32_t n_blocks, uint64_t key,
                    uint32_t lo, uint32_t hi, hipStream_t stream) {
  int64_t n = nrows * n_blocks;
  if (n <= 0) return 0;
  if (hi < lo || hi > 255u) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(k_fill_e8m0, dim3(grid_for(n, 256)), dim3(256), 0, stream, dst,
                     row0 * n_blocks, n, key, lo, hi - lo + 1u);
  return int(hipGetLastError());
}

// Fills elements [i0, i0 + n) of an approximately-normal bf16 tensor; dst points at element i0.
int synth_fill_normal_bf16(uint16_t* dst, int64_t i0, int64_t n, uint64_t key, double mean,
                           double stdv, hipStream_t stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fill_normal_bf16, dim3(grid_for(n, 256)), dim3(256), 0, stream, dst, i0,
                     n, key, mean, stdv);
  return int(hipGetLastError());
}

// Fills the residual streams of tokens [tok0, tok0 + ntok); per_tok = hc * dim elements each.
int synth_fill_x(uint16_t* dst, int64_t tok0, int64_t ntok, int64_t per_tok, uint64_t key_x,
                 uint64_t key_outlier, uint32_t thr, double stdv, double outlier_std,
                 hipStream_t stream) {
  int64_t n = ntok * per_tok;
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fill_x, dim3(grid_for(n, 256)), dim3(256), 0, stream, dst, tok0, ntok,
                     per_tok, key_x, key_outlier, thr, stdv, outlier_std);
  return int(hipGetLastError());
}

}  // extern "C"
