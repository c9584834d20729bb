// Standalone kernels: row gather + dequantisation, and gate + residual add from a given kv.
#include "common.h"
#include "launch.h"

namespace engram {

// ----------------------------------------------------------------------------------------
// Row gather and dequantisation (engram-second page, ParallelEngramEmbedding.forward with one
// shard, flattened as in Engram.forward).  One thread per 16 codes of one gathered row:
// a 16-byte load of codes, one scale (fp32, or an E8M0 byte), two 16-byte stores of bf16.
// ----------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gather_dequant(GatherArgs a) {
  const int chunks = a.head_dim >> 4;
  const int nb = a.head_dim / a.scale_block;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t pair = gid / chunks;  // flat (token, column) index m * n_cols + j
  const int ch = int(gid - pair * chunks);
  const bool fill = a.frag_cols > 0 && pair >= a.n_pairs;  // a zero row past the last token
  if (pair >= a.n_pairs && !(fill && pair < a.n_fill)) return;
  const int64_t r = fill ? -1 : a.hash_ids[pair];
  u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = {0u, 0u, 0u, 0u};
  if (fill) {
  } else if (r >= 0 && r < a.n_rows) {
    const u32x4 c = *reinterpret_cast<const u32x4*>(a.table + r * a.head_dim + ch * 16);
    const float s = load_scale(a.scales, r * nb + (ch * 16) / a.scale_block, a.scale_e8m0);
    dequant16(c, s, o0, o1);
  } else if (ch == 0 && a.err_count != nullptr) {
    atomicAdd(a.err_count, 1);
  }
  if (a.frag_cols > 0) {
    // features f .. f + 15 of token m: two 8-feature pieces, each lane (m % 16) + 16 q of the
    // 1 KB block (m / 16, f / 32), q = (f / 8) % 4
    const int64_t m = pair / a.frag_cols;
    const int64_t f = (pair - m * a.frag_cols) * a.head_dim + ch * 16;
    const int64_t k32 = int64_t(a.frag_cols) * a.head_dim / 32;
    u32x4* const blk = reinterpret_cast<u32x4*>(a.emb) + ((m >> 4) * k32 + (f >> 5)) * 64 + (m & 15);
    const int q = int(f >> 3) & 3;
    blk[16 * q] = o0;
    blk[16 * (q + 1)] = o1;
    return;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(a.emb + pair * a.head_dim + ch * 16);
  dst[0] = o0;
  dst[1] = o1;
}

// ----------------------------------------------------------------------------------------
// Gate and residual add from kv (engram-second page, Engram.forward after the projection).
// One 256-thread workgroup per token.  Pass 1 accumulates, per stream, sum h^2, sum key^2 and
// sum h*w*key over chunks of 8 features; the sums are reduced in a fixed order (in-thread, then
// butterfly within the wave, then the four waves in order), so results are deterministic.
// Pass 2 re-reads x (cache-resident) and writes bf16(h + g * value).
// ----------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gate_apply(GateArgs a) {
  __shared__ float s_part[4][12];
  __shared__ float s_gate[4];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int dim = a.dim;
  const int nch = dim >> 3;
  const uint16_t* xm = a.x + m * int64_t(4 * dim);
  const uint16_t* kvm = a.kv + m * int64_t(5 * dim);
  uint16_t* om = a.out + m * int64_t(4 * dim);
  const bool open = a.token_mask == nullptr || a.token_mask[m] != 0;

  if (!open) {  // closed gate: the token passes through untouched
    if (om != xm)
      for (int c = tid; c < 4 * nch; c += 256)
        reinterpret_cast<u32x4*>(om)[c] = reinterpret_cast<const u32x4*>(xm)[c];
    if (a.gate != nullptr && tid < 4) a.gate[m * 4 + tid] = 0.0f;
    return;
  }

  float A[4] = {0.f, 0.f, 0.f, 0.f}, Kq[4] = {0.f, 0.f, 0.f, 0.f}, D[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c = tid; c < nch; c += 256) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(xm + s * dim + 8 * c);
      const u32x4 kv = *reinterpret_cast<const u32x4*>(kvm + s * dim + 8 * c);
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(a.q_weight + s * dim + 8 * c);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(a.q_weight + s * dim + 8 * c + 4);
      const f32x4 k0 = *reinterpret_cast<const f32x4*>(a.k_weight + s * dim + 8 * c);
      const f32x4 k1 = *reinterpret_cast<const f32x4*>(a.k_weight + s * dim + 8 * c + 4);
      const float qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float h = (e & 1) ? bf16_hi(xw[e >> 1]) : bf16_lo(xw[e >> 1]);
        const float key = (e & 1) ? bf16_hi(kw[e >> 1]) : bf16_lo(kw[e >> 1]);
        const float w = qq[e] * kk[e];
        A[s] += h * h;
        Kq[s] += key * key;
        D[s] += (h * w) * key;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    A[s] = wave_sum(A[s]);
    Kq[s] = wave_sum(Kq[s]);
    D[s] = wave_sum(D[s]);
  }
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      s_part[wv][3 * s + 0] = A[s];
      s_part[wv][3 * s + 1] = Kq[s];
      s_part[wv][3 * s + 2] = D[s];
    }
  }
  __syncthreads();
  if (tid < 4) {
    const int s = tid;
    float sa = 0.f, sk = 0.f, sd = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sa += s_part[w][3 * s + 0];
      sk += s_part[w][3 * s + 1];
      sd += s_part[w][3 * s + 2];
    }
    const float fd = float(dim);
    const float rstd = __frsqrt_rn(sa / fd + a.eps) * __frsqrt_rn(sk / fd + a.eps);
    const float dot = sd * rstd * a.inv_sqrt_dim;
    const float z = copysignf(sqrtf(fmaxf(fabsf(dot), a.clamp)), dot);
    const float g = 1.0f / (1.0f + expf(-z));
    s_gate[s] = g;
    if (a.gate != nullptr) a.gate[m * 4 + s] = g;
  }
  __syncthreads();
  const float g0 = s_gate[0], g1 = s_gate[1], g2 = s_gate[2], g3 = s_gate[3];
  for (int c = tid; c < nch; c += 256) {
    const u32x4 vv = *reinterpret_cast<const u32x4*>(kvm + 4 * dim + 8 * c);
    const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float g = s == 0 ? g0 : (s == 1 ? g1 : (s == 2 ? g2 : g3));
      const u32x4 xv = *reinterpret_cast<const u32x4*>(xm + s * dim + 8 * c);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      uint32_t ow[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
        ow[p] = pack_bf16x2(bf16_lo(xw[p]) + g * bf16_lo(vw[p]), bf16_hi(xw[p]) + g * bf16_hi(vw[p]));
      *reinterpret_cast<u32x4*>(om + s * dim + 8 * c) = u32x4{ow[0], ow[1], ow[2], ow[3]};
    }
  }
}

// ----------------------------------------------------------------------------------------
// Row gather without dequantisation, for the fp8 tiled schedule (E8M0 table scales): the codes
// as they are and one E8M0 byte per 32 features (a table scale covers scale_block / 32 of
// them).  One thread per 16 codes; the even ones also write their 32-feature block's scale.
// ----------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gather_mx(GatherArgs a, uint8_t* codes8, uint8_t* scales8) {
  const int chunks = a.head_dim >> 4;
  const int nb = a.head_dim / a.scale_block;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t pair = gid / chunks;
  const int ch = int(gid - pair * chunks);
  if (pair >= a.n_pairs) return;
  const int64_t r = a.hash_ids[pair];
  const bool ok = r >= 0 && r < a.n_rows;
  u32x4 c = {0u, 0u, 0u, 0u};
  uint8_t sc = 127;
  if (ok) {
    c = *reinterpret_cast<const u32x4*>(a.table + r * a.head_dim + ch * 16);
    sc = static_cast<const uint8_t*>(a.scales)[r * nb + (ch * 16) / a.scale_block];
  } else if (ch == 0 && a.err_count != nullptr) {
    atomicAdd(a.err_count, 1);
  }
  *reinterpret_cast<u32x4*>(codes8 + pair * a.head_dim + ch * 16) = c;
  if ((ch & 1) == 0) scales8[pair * (a.head_dim / 32) + ch / 2] = sc;
}

hipError_t launch_gather_mx(const GatherArgs& a, uint8_t* codes8, uint8_t* scales8, hipStream_t stream) {
  const int64_t threads = a.n_pairs * (a.head_dim >> 4);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(k_gather_mx, dim3(unsigned(blocks)), dim3(256), 0, stream, a, codes8, scales8);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// MXFP8 weights -> bf16 (for the schedules that stream bf16 weights): one thread per 16
// codes of a row, which share one E8M0 scale (16-aligned pieces of 32-feature blocks).
// ----------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_expand_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t n16,
                                                       int K, uint16_t* out) {
  const int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= n16) return;
  const int64_t e = g * 16;  // flat element index n * K + k
  const int64_t n = e / K;
  const int64_t k = e - n * K;
  const u32x4 c = *reinterpret_cast<const u32x4*>(codes + e);
  u32x4 o0, o1;
  dequant16(c, e8m0_to_f32(scales[n * (K / 32) + k / 32]), o0, o1);
  u32x4* dst = reinterpret_cast<u32x4*>(out + e);
  dst[0] = o0;
  dst[1] = o1;
}

hipError_t launch_expand_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t N, int K, uint16_t* out,
                               hipStream_t stream) {
  const int64_t n16 = N * K / 16;
  const int64_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(k_expand_mxfp8, dim3(unsigned(blocks)), dim3(256), 0, stream, codes, scales, n16, K, out);
  return hipGetLastError();
}

hipError_t launch_gather_dequant(const GatherArgs& a, hipStream_t stream) {
  const int64_t pairs = a.frag_cols > 0 && a.n_fill > a.n_pairs ? a.n_fill : a.n_pairs;
  const int64_t threads = pairs * (a.head_dim >> 4);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(k_gather_dequant, dim3(unsigned(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gate_apply(const GateArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_gate_apply, dim3(unsigned(a.M)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace engram
