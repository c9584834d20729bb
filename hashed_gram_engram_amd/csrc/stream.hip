// Weight-streaming wkv projection for small token counts (decode), alone or fused with the
// row gather, the per-stream gate and the residual add.
//
// Schedule.  The N = (hc + 1) * dim output columns are cut into 16-column row blocks of the
// wkv matrix ([N, K], K contiguous).  A persistent grid of G workgroups (one per CU) gives
// workgroup w the contiguous row blocks [w * nrb / G, (w + 1) * nrb / G), so every byte of wkv
// is read exactly once per 64-token block and the load is balanced to within one row block.
// Each of the four waves of a workgroup owns one 32-feature slice of every 128-feature chunk
// of K (a split of K inside the workgroup), streams its weight fragments straight from HBM into
// registers (no LDS, no reuse needed) with a ring of PF chunks in flight, and multiplies them
// against the token tile held in LDS.  The token tile (64 tokens x 128 features, bf16) is
// double buffered; in the fused kernel it is produced by gathering the fp8 rows of the hash
// ids and dequantising them on the way into LDS.  At the end the four K-partials are summed in
// a fixed order through LDS.
//
// MFMA roles: the weight rows are the A operand (16 rows), the tokens the B operand (16 tokens),
// so every lane ends up holding four consecutive output columns of one token.
//
// Fused epilogue.  Key columns of stream s contribute, per token, partial sums of h^2, key^2
// and h * q * k * key over their features; each workgroup posts one partial per (token,
// stream) and bumps a per-stream counter.  The workgroup that arrives last for a stream sums
// the partials of all contributing workgroups in workgroup order (deterministic), evaluates
// the gate of the 64 tokens and raises a flag.  Workgroups holding value columns wait for the
// four flags, then write out = bf16(h + g * value) for their features on all four streams.
// Only value workgroups ever wait and they wait on work that never waits, so the grid cannot
// deadlock once all workgroups are resident (cooperative launch); every wait is bounded.
#include "common.h"
#include "launch.h"

namespace engram {

namespace {

constexpr int kTB = 64;        // tokens per token block
constexpr int kKC = 128;       // features per K chunk (4 waves x 32)
constexpr int kLdsRow = kKC + 8;  // padded LDS row (bf16 elements) against bank conflicts

__device__ __forceinline__ int rb_begin(int w, int nrb, int G) { return int(int64_t(w) * nrb / G); }
// workgroup that owns row block rb
__device__ __forceinline__ int owner_of_rb(int rb, int nrb, int G) {
  return int((int64_t(rb + 1) * G - 1) / nrb);
}

template <bool FUSED>
struct TileLoader {
  // two 16-feature groups per thread per chunk
  u32x4 c[2];
  u32x4 c2[2];
  float s[2];
  bool ok[2];

  __device__ __forceinline__ void load(const StreamArgs& a, int64_t m0, int chunk, int tid) {
    const int grp = tid & 7;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tok = (tid >> 3) + 32 * i;
      const int64_t m = m0 + tok;
      const int f = chunk * kKC + 16 * grp;
      ok[i] = false;
      c[i] = u32x4{0u, 0u, 0u, 0u};
      c2[i] = u32x4{0u, 0u, 0u, 0u};
      s[i] = 0.0f;
      if (m < a.M) {
        if constexpr (FUSED) {
          const int j = f / a.head_dim;
          const int cc = f - j * a.head_dim;
          const int64_t r = a.hash_ids[m * a.n_cols + j];
          if (r >= 0 && r < a.n_rows) {
            ok[i] = true;
            c[i] = *reinterpret_cast<const u32x4*>(a.table + r * a.head_dim + cc);
            s[i] = a.scales[r * (a.head_dim / a.scale_block) + cc / a.scale_block];
          } else if (cc == 0 && blockIdx.x == 0 && a.err_count != nullptr) {
            atomicAdd(a.err_count, 1);
          }
        } else {
          const u32x4* src = reinterpret_cast<const u32x4*>(a.emb + m * a.K + f);
          c[i] = src[0];
          c2[i] = src[1];
          ok[i] = true;
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* buf, int tid) {
    const int grp = tid & 7;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tok = (tid >> 3) + 32 * i;
      u32x4 o0 = c[i], o1 = c2[i];
      if constexpr (FUSED) {
        if (ok[i]) {
          dequant16(c[i], s[i], o0, o1);
        } else {
          o0 = u32x4{0u, 0u, 0u, 0u};
          o1 = o0;
        }
      }
      u32x4* dst = reinterpret_cast<u32x4*>(buf + tok * kLdsRow + 16 * grp);
      dst[0] = o0;
      dst[1] = o1;
    }
  }
};

template <int NRB>
__device__ __forceinline__ void load_weights(u32x4 (&wb)[NRB], const StreamArgs& a, int rb0, int cnt,
                                             int chunk, int lane, int wv) {
  const size_t col = size_t(chunk) * kKC + 32 * wv + 8 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < NRB; ++i) {
    if (i < cnt) {
      const size_t row = size_t(rb0 + i) * 16 + (lane & 15);
      wb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.wkv + row * a.K + col));
    }
  }
}

template <int NRB, int PF, bool FUSED>
__global__ __launch_bounds__(256, 1) void k_stream(StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ float s_red[4][kTB][3];
  __shared__ int s_last[2];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = gridDim.x, w = blockIdx.x;
  const int nrb = a.N >> 4;
  const int rb0 = rb_begin(w, nrb, G);
  const int cnt = rb_begin(w + 1, nrb, G) - rb0;
  const int nchunk = a.K / kKC;
  const int64_t n_tb = (a.M + kTB - 1) / kTB;
  const int R = a.dim >> 4;  // row blocks per stream segment
  const int seg_lo = rb0 / R;
  const int seg_hi = (rb0 + cnt - 1) / R;

  uint16_t* const lds_tiles = reinterpret_cast<uint16_t*>(smem);  // two token tiles

  for (int64_t tb = 0; tb < n_tb; ++tb) {
    const int64_t m0 = tb * kTB;
    f32x4 acc[NRB][4];
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wb[PF][NRB];
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < nchunk) load_weights<NRB>(wb[p], a, rb0, cnt, p, lane, wv);

    TileLoader<FUSED> tl;
    tl.load(a, m0, 0, tid);
    tl.store(lds_tiles, tid);
    __syncthreads();

    for (int c0 = 0; c0 < nchunk; c0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        const int c = c0 + p;
        if (c < nchunk) {
          if (c + 1 < nchunk) tl.load(a, m0, c + 1, tid);
          const uint16_t* buf = lds_tiles + (c & 1) * (kTB * kLdsRow);
          u32x4 bt[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            bt[t] = *reinterpret_cast<const u32x4*>(buf + (16 * t + (lane & 15)) * kLdsRow + 32 * wv +
                                                    8 * (lane >> 4));
#pragma unroll
          for (int i = 0; i < NRB; ++i)
            if (i < cnt)
#pragma unroll
              for (int t = 0; t < 4; ++t) acc[i][t] = mfma16x16x32(wb[p][i], bt[t], acc[i][t]);
          if (c + PF < nchunk) load_weights<NRB>(wb[p], a, rb0, cnt, c + PF, lane, wv);
          if (c + 1 < nchunk) tl.store(lds_tiles + ((c + 1) & 1) * (kTB * kLdsRow), tid);
          __syncthreads();
        }
      }
    }

    // ---- sum the four K-partials in wave order; wave wv keeps token sub-block wv
    f32x4 red[NRB];
    f32x4* X = reinterpret_cast<f32x4*>(smem);  // [4 waves][2][4 sub-blocks][64 lanes]
#pragma unroll
    for (int r0 = 0; r0 < NRB; r0 += 2) {
      if (r0 < cnt) {
        __syncthreads();
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
          if (r0 + ii < NRB && r0 + ii < cnt)
#pragma unroll
            for (int t = 0; t < 4; ++t) X[((wv * 2 + ii) * 4 + t) * 64 + lane] = acc[r0 + ii][t];
        __syncthreads();
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
          if (r0 + ii < NRB && r0 + ii < cnt) {
            f32x4 s = X[((0 * 2 + ii) * 4 + wv) * 64 + lane];
            s += X[((1 * 2 + ii) * 4 + wv) * 64 + lane];
            s += X[((2 * 2 + ii) * 4 + wv) * 64 + lane];
            s += X[((3 * 2 + ii) * 4 + wv) * 64 + lane];
            red[r0 + ii] = s;
          }
      }
    }

    const int tok = 16 * wv + (lane & 15);
    const int64_t m = m0 + tok;
    const bool mvalid = m < a.M;

    if constexpr (!FUSED) {
      if (mvalid) {
#pragma unroll
        for (int i = 0; i < NRB; ++i)
          if (i < cnt) {
            const int n = (rb0 + i) * 16 + 4 * (lane >> 4);
            *reinterpret_cast<u32x2*>(a.kv + m * a.N + n) =
                u32x2{pack_bf16x2(red[i].x, red[i].y), pack_bf16x2(red[i].z, red[i].w)};
          }
      }
      __syncthreads();
    } else {
      // ---- key columns: per-token partial sums for up to two streams
      float pa[2] = {0.f, 0.f}, pk[2] = {0.f, 0.f}, pd[2] = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NRB; ++i) {
        if (i < cnt) {
          const int rb = rb0 + i;
          const int s = rb / R;
          if (s < 4) {
            const int d = (rb - s * R) * 16 + 4 * (lane >> 4);
            const float key[4] = {bf16_round(red[i].x), bf16_round(red[i].y), bf16_round(red[i].z),
                                  bf16_round(red[i].w)};
            u32x2 xw = {0u, 0u};
            if (mvalid) xw = *reinterpret_cast<const u32x2*>(a.x + (m * 4 + s) * a.dim + d);
            const f32x4 q4 = *reinterpret_cast<const f32x4*>(a.q_weight + s * a.dim + d);
            const f32x4 k4 = *reinterpret_cast<const f32x4*>(a.k_weight + s * a.dim + d);
            const float h[4] = {bf16_lo(xw.x), bf16_hi(xw.x), bf16_lo(xw.y), bf16_hi(xw.y)};
            const float wq[4] = {q4.x * k4.x, q4.y * k4.y, q4.z * k4.z, q4.w * k4.w};
            float sa = 0.f, sk = 0.f, sd = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              sa += h[r] * h[r];
              sk += key[r] * key[r];
              sd += (h[r] * wq[r]) * key[r];
            }
            const int slot = s - seg_lo;
            if (slot == 0) {
              pa[0] += sa; pk[0] += sk; pd[0] += sd;
            } else {
              pa[1] += sa; pk[1] += sk; pd[1] += sd;
            }
          }
        }
      }
      if (seg_lo < 4) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          pa[sl] += __shfl_xor(pa[sl], 16, 64); pa[sl] += __shfl_xor(pa[sl], 32, 64);
          pk[sl] += __shfl_xor(pk[sl], 16, 64); pk[sl] += __shfl_xor(pk[sl], 32, 64);
          pd[sl] += __shfl_xor(pd[sl], 16, 64); pd[sl] += __shfl_xor(pd[sl], 32, 64);
        }
        if (lane < 16) {
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) {
            if (seg_lo + sl <= seg_hi && seg_lo + sl < 4) {
              float* P = a.partials + ((size_t(tb) * G + w) * 2 + sl) * (kTB * 3) + tok * 3;
              P[0] = pa[sl];
              P[1] = pk[sl];
              P[2] = pd[sl];
            }
          }
        }
        fence_release_agent();
        __syncthreads();
        if (tid == 0) {
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) {
            const int s = seg_lo + sl;
            s_last[sl] = 0;
            if (s <= seg_hi && s < 4) {
              const int wf = owner_of_rb(s * R, nrb, G), wl = owner_of_rb((s + 1) * R - 1, nrb, G);
              const uint32_t old = atomic_add_relaxed(&a.counters[tb * 4 + s], 1u);
              s_last[sl] = (old == uint32_t(wl - wf)) ? 1 : 0;
            }
          }
        }
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          if (s_last[sl]) {
            fence_acquire_agent();
            const int s = seg_lo + sl;
            const int wf = owner_of_rb(s * R, nrb, G), wl = owner_of_rb((s + 1) * R - 1, nrb, G);
            const int nW = wl - wf + 1;
            const int t = tid & 63, q = tid >> 6;
            const int wb0 = wf + (nW * q) / 4, wb1 = wf + (nW * (q + 1)) / 4;
            float ra = 0.f, rk = 0.f, rd = 0.f;
            for (int w2 = wb0; w2 < wb1; ++w2) {
              const int sl2 = s - rb_begin(w2, nrb, G) / R;
              const float* P = a.partials + ((size_t(tb) * G + w2) * 2 + sl2) * (kTB * 3) + t * 3;
              ra += P[0];
              rk += P[1];
              rd += P[2];
            }
            s_red[q][t][0] = ra;
            s_red[q][t][1] = rk;
            s_red[q][t][2] = rd;
            __syncthreads();
            if (q == 0) {
              const float A = ((s_red[0][t][0] + s_red[1][t][0]) + s_red[2][t][0]) + s_red[3][t][0];
              const float Kq = ((s_red[0][t][1] + s_red[1][t][1]) + s_red[2][t][1]) + s_red[3][t][1];
              const float D = ((s_red[0][t][2] + s_red[1][t][2]) + s_red[2][t][2]) + s_red[3][t][2];
              const float fd = float(a.dim);
              const float rstd = __frsqrt_rn(A / fd + a.eps) * __frsqrt_rn(Kq / fd + a.eps);
              const float dot = D * rstd * a.inv_sqrt_dim;
              const float z = copysignf(sqrtf(fmaxf(fabsf(dot), a.clamp)), dot);
              float g = 1.0f / (1.0f + expf(-z));
              const int64_t mt = m0 + t;
              const bool open = mt < a.M && (a.token_mask == nullptr || a.token_mask[mt] != 0);
              a.gates[(size_t(tb) * 4 + s) * kTB + t] = open ? g : 0.0f;
              fence_release_agent();
            }
            __syncthreads();
            if (tid == 0)
              __hip_atomic_store(&a.flags[tb * 4 + s], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }

      // ---- value columns: wait for the four gates, then out = h + g * value on every stream
      if (seg_hi == 4) {
        if (tid == 0) {
          bool ok = true;
#pragma unroll
          for (int s = 0; s < 4; ++s) ok = ok && wait_at_least(&a.flags[tb * 4 + s], 1u, a.spin_budget);
          if (!ok) atomic_add_relaxed(&a.ws_hdr[0], 1u);
        }
        __syncthreads();
        fence_acquire_agent();
        float g[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) g[s] = a.gates[(size_t(tb) * 4 + s) * kTB + tok];
        const bool open = mvalid && (a.token_mask == nullptr || a.token_mask[m] != 0);
        if (mvalid) {
#pragma unroll
          for (int i = 0; i < NRB; ++i) {
            if (i < cnt && (rb0 + i) / R == 4) {
              const int d = (rb0 + i - 4 * R) * 16 + 4 * (lane >> 4);
              const float v[4] = {bf16_round(red[i].x), bf16_round(red[i].y), bf16_round(red[i].z),
                                  bf16_round(red[i].w)};
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                const size_t off = size_t(m * 4 + s) * a.dim + d;
                const u32x2 xw = *reinterpret_cast<const u32x2*>(a.x + off);
                u32x2 o = xw;
                if (open) {
                  o.x = pack_bf16x2(bf16_lo(xw.x) + g[s] * v[0], bf16_hi(xw.x) + g[s] * v[1]);
                  o.y = pack_bf16x2(bf16_lo(xw.y) + g[s] * v[2], bf16_hi(xw.y) + g[s] * v[3]);
                }
                if (open || a.out != a.x) *reinterpret_cast<u32x2*>(a.out + off) = o;
              }
            }
          }
        }
      }
      __syncthreads();
    }
  }

  if constexpr (FUSED) {
    // last workgroup out leaves the counters and flags zeroed for the next call
    fence_release_agent();
    __syncthreads();
    if (tid == 0) s_last[0] = (atomic_add_relaxed(&a.ws_hdr[1], 1u) == uint32_t(G - 1)) ? 1 : 0;
    __syncthreads();
    if (s_last[0]) {
      fence_acquire_agent();
      for (int64_t i = tid; i < n_tb * 4; i += 256) {
        store_relaxed(&a.counters[i], 0u);
        store_relaxed(&a.flags[i], 0u);
      }
      if (tid == 0) store_relaxed(&a.ws_hdr[1], 0u);
    }
  }
}

constexpr size_t kDynLds = size_t(2) * kTB * kLdsRow * 2;  // two bf16 token tiles (also holds
                                                          // the 32 KB reduction buffer)
static_assert(size_t(4) * 2 * 4 * 64 * 16 <= kDynLds, "reduction buffer must fit");

template <bool FUSED>
hipError_t launch_stream_impl(const StreamArgs& a, int G, int per_wg, hipStream_t stream, bool coop) {
  void* fn = nullptr;
  if (per_wg <= 1) fn = reinterpret_cast<void*>(&k_stream<1, 3, FUSED>);
  else if (per_wg <= 2) fn = reinterpret_cast<void*>(&k_stream<2, 3, FUSED>);
  else if (per_wg <= 4) fn = reinterpret_cast<void*>(&k_stream<4, 3, FUSED>);
  else if (per_wg <= 8) fn = reinterpret_cast<void*>(&k_stream<8, 2, FUSED>);
  else return hipErrorInvalidValue;
  StreamArgs arg = a;
  void* params[] = {&arg};
  if (coop)
    return hipLaunchCooperativeKernel(fn, dim3(G), dim3(256), params, unsigned(kDynLds), stream);
  return hipLaunchKernel(fn, dim3(G), dim3(256), params, kDynLds, stream);
}

}  // namespace

int stream_grid(int N, int num_cus) {
  const int nrb = N / 16;
  int G = num_cus;
  if (G > nrb) G = nrb;
  while ((nrb + G - 1) / G > 8) ++G;  // at most 8 row blocks per workgroup
  return G;
}

size_t stream_workspace_bytes(int64_t M, int N, int grid) {
  const int64_t n_tb = (M + kTB - 1) / kTB;
  size_t b = 256;                              // header
  b += size_t(n_tb) * 4 * 4 * 2;               // counters + flags
  b = (b + 255) & ~size_t(255);
  b += size_t(n_tb) * 4 * kTB * 4;             // gates
  b += size_t(n_tb) * grid * 2 * kTB * 3 * 4;  // partials
  (void)N;
  return b;
}

hipError_t launch_kv_proj_stream(const StreamArgs& a, int num_cus, hipStream_t stream) {
  const int G = stream_grid(a.N, num_cus);
  const int nrb = a.N / 16;
  return launch_stream_impl<false>(a, G, (nrb + G - 1) / G, stream, false);
}

hipError_t launch_forward_stream(StreamArgs a, void* workspace, int num_cus, hipStream_t stream) {
  const int G = stream_grid(a.N, num_cus);
  const int nrb = a.N / 16;
  const int64_t n_tb = (a.M + kTB - 1) / kTB;
  char* ws = static_cast<char*>(workspace);
  a.ws_hdr = reinterpret_cast<uint32_t*>(ws);
  a.counters = reinterpret_cast<uint32_t*>(ws + 256);
  a.flags = a.counters + n_tb * 4;
  size_t off = 256 + size_t(n_tb) * 4 * 4 * 2;
  off = (off + 255) & ~size_t(255);
  a.gates = reinterpret_cast<float*>(ws + off);
  off += size_t(n_tb) * 4 * kTB * 4;
  a.partials = reinterpret_cast<float*>(ws + off);
  return launch_stream_impl<true>(a, G, (nrb + G - 1) / G, stream, true);
}

}  // namespace engram
