// Tiled wkv projection for large token counts (prefill), alone or fused with the row gather,
// the per-stream gate and the residual add.
//
// A workgroup computes one tile of 256 tokens x 256 wkv rows (output columns) over all of K, in
// steps of 64 features.  Each step's two operands sit in LDS as 256 rows of 128 bytes with an
// XOR swizzle of 16-byte chunks (double buffered, 128 KB); while step k is multiplied, step
// k + 1 is loaded.  Eight waves (two per SIMD, so one can issue MFMAs while the other waits
// at a barrier or on LDS) each own 128 columns x 64 tokens: 8 x 4 blocks of
// v_mfma_f32_16x16x32_bf16, 128 accumulator registers.  The wkv rows are the A operand and the
// tokens the B operand, so a lane ends up holding four consecutive output columns of one token.
//
// Operand loads: wkv rows (and, for the projection alone, the dense bf16 tokens) are copied
// from global memory straight into LDS (global_load_lds_dwordx4, 8 rows of 128 bytes per wave
// instruction), so they take no registers.  In the fused kernel a step's 64 features of a token
// lie in one hash column (head_dim is a multiple of 64): 4 lanes per token gather 16 fp8 codes
// each from the token's table row, dequantise them with the row's block scale and write bf16 to
// LDS.  The hash ids of step k + 2 are loaded during step k, so no gather address waits on a
// load issued in the same step.
//
// Tile order: workgroup b takes token block b % n_tb and column block b / n_tb, so the tiles
// resident at one time share weight panels across token blocks, and (workgroups being dealt
// to the 8 XCDs round robin) all tiles of a token block run on one XCD when n_tb is a multiple
// of 8, keeping its gathered rows and its x in that XCD's L2.  In the fused kernel every key
// column block comes before every value column block.  Key tiles post per-(token, stream)
// partial sums of the gate's three reductions; the last key tile of each (token block, stream)
// sums them in column-block order, evaluates the gates and hands them to the value tiles of the
// token block through per-tile slots.  A value tile waits only on key tiles with lower ids,
// which never wait, and every wait is bounded (time-outs are counted in workspace word 0).
#include "common.h"
#include "launch.h"

namespace engram {

namespace {

constexpr int kThreads = 512;           // 8 waves
constexpr int kTM = 256;                // tokens per tile
constexpr int kTN = 256;                // wkv rows per tile
constexpr int kTK = 64;                 // features per K step
constexpr int kRowB = kTK * 2;          // bytes per LDS row: 8 chunks of 16 bytes
constexpr int kOp = 256 * kRowB;        // one operand of one stage (32 KB)
constexpr int kStage = 2 * kOp;         // wkv rows + tokens
constexpr int kLds = 2 * kStage;        // double buffer: 128 KB
constexpr int kBI = 8;                  // 16-column blocks per wave
constexpr int kBJ = 4;                  // 16-token blocks per wave

typedef f32x4 TileAcc[kBI][kBJ];

// LDS rows are stored with 16-byte chunk c of row r at position c ^ (r & 7): the eight rows that
// one 8-lane phase of a 16-byte LDS read touches then hit eight distinct bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowB + 16 * (chunk ^ (row & 7)); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Direct global -> LDS copy of 256 rows x 128 bytes (features k0 .. k0 + 63 of rows
// row0 .. row0 + 255 of a row-major bf16 matrix with ld elements per row; rows past row_last
// repeat row_last).  Each wave instruction fills 1024 contiguous LDS bytes (lane l at 16 l),
// i.e. 8 rows: lane l supplies chunk (l & 7) ^ (l >> 3) of row l >> 3 of its group, which is
// the swizzled position (l & 7).  Wave w fills the row groups 4 w .. 4 w + 3.
__device__ __forceinline__ void dma_rows(const uint16_t* src, int64_t ld, int64_t row0, int64_t row_last, int k0,
                                         char* dst, int wv_u, int lane) {
  const int r = lane >> 3, c = (lane & 7) ^ r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = wv_u * 4 + i;  // 8-row group 0..31 (wave-uniform)
    int64_t row = row0 + 8 * g + r;
    row = row < row_last ? row : row_last;
    __builtin_amdgcn_global_load_lds((const void*)(src + row * ld + k0 + 8 * c), (lds_ptr_t)(dst + g * 1024), 16,
                                     0, 0);
  }
}

struct TiledIds {
  int64_t r[2];    // hash id of token (tid >> 2) + 128 i for one column (of the last token for
                   // positions past it: validity is decided where the ids are used)
};

struct TiledCodes {
  u32x4 c[2];      // 16 fp8 codes of token (tid >> 2) + 128 i at features 16 (tid & 3) of the step
  float scale[2];  // their block scale
  uint32_t keep[2];
};

__device__ __forceinline__ void issue_ids(TiledIds& ids, const TiledArgs& a, int64_t m0, int k0, int tid) {
  const int j = k0 / a.head_dim;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + (tid >> 2) + 128 * i;
    const int64_t mm = m < a.M ? m : a.M - 1;
    ids.r[i] = a.hash_ids[mm * a.n_cols + j];
  }
}

__device__ __forceinline__ void issue_codes(TiledCodes& st, const TiledIds& ids, const TiledArgs& a, int64_t m0,
                                            int k0, int tid) {
  const int j = k0 / a.head_dim;
  const int cc = k0 - j * a.head_dim + 16 * (tid & 3);
  const int nb = a.head_dim / a.scale_block;
  const int sb = cc / a.scale_block;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t r = ids.r[i];
    const bool ok = m0 + (tid >> 2) + 128 * i < a.M && r >= 0 && r < a.n_rows;
    const int64_t rr = ok ? r : 0;
    st.keep[i] = ok ? 0xFFFFFFFFu : 0u;
    st.c[i] = *reinterpret_cast<const u32x4*>(a.table + rr * a.head_dim + cc);
    st.scale[i] = a.scales[rr * nb + sb];
  }
}

// Dequantised tokens of one step into the token operand of a stage (bf16, swizzled rows).
__device__ __forceinline__ void store_codes(const TiledCodes& st, char* T, int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x4 c = st.c[i];
    const uint32_t k = st.keep[i];
    const float s = st.scale[i];
    const u32x2 p0 = dequant4_raw(c.x, s), p1 = dequant4_raw(c.y, s);
    const u32x2 p2 = dequant4_raw(c.z, s), p3 = dequant4_raw(c.w, s);
    const int row = (tid >> 2) + 128 * i, ch = 2 * (tid & 3);
    *reinterpret_cast<u32x4*>(T + swz(row, ch)) = u32x4{p0.x & k, p0.y & k, p1.x & k, p1.y & k};
    *reinterpret_cast<u32x4*>(T + swz(row, ch + 1)) = u32x4{p2.x & k, p2.y & k, p3.x & k, p3.y & k};
  }
}

// The 64 features of one stage: two k32 steps of 8 x 4 MFMA blocks per wave.
__device__ __forceinline__ void stage_mma(TileAcc& acc, const char* stage, int lane, int wr, int wt) {
  const char* W = stage + (128 * wr) * kRowB;
  const char* T = stage + kOp + (64 * wt) * kRowB;
  const int r = lane & 15;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int ch = 4 * s + (lane >> 4);
    u32x4 af[kBI], bf[kBJ];
#pragma unroll
    for (int i = 0; i < kBI; ++i) af[i] = *reinterpret_cast<const u32x4*>(W + swz(16 * i + r, ch));
#pragma unroll
    for (int j = 0; j < kBJ; ++j) bf[j] = *reinterpret_cast<const u32x4*>(T + swz(16 * j + r, ch));
#pragma unroll
    for (int i = 0; i < kBI; ++i)
#pragma unroll
      for (int j = 0; j < kBJ; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
  }
}

// Every load of this wave has landed (registers and LDS) and every LDS access is done; then the
// workgroup barrier.  (A plain barrier: LDS needs no cache maintenance.)
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Operand loads of the step at feature k0 into stage buffer `stage`.  The fused kernel's token
// operand goes through registers: the codes are gathered here (with the hash ids loaded one
// step earlier), the ids of the step after are loaded, and store_codes writes the tokens later.
// The gathers come first, so that the wait for the ids they use is a wait for loads issued
// before the previous barrier, never for the copies issued here.
template <bool FUSED>
__device__ __forceinline__ void issue_step(TiledCodes& codes, TiledIds& ids, const TiledArgs& a, char* stage,
                                           int64_t m0, int n0, int k0, int k0_ids, int wv_u, int lane, int tid) {
  if constexpr (FUSED) {
    issue_codes(codes, ids, a, m0, k0, tid);
    issue_ids(ids, a, m0, k0_ids, tid);
  }
  dma_rows(a.wkv, a.K, n0, int64_t(n0) + kTN - 1, k0, stage, wv_u, lane);
  if constexpr (!FUSED) dma_rows(a.emb, a.K, m0, a.M - 1, k0, stage + kOp, wv_u, lane);
}

template <bool FUSED>
__device__ __forceinline__ void tiled_gemm(TileAcc& acc, const TiledArgs& a, char* lds, int64_t m0, int n0,
                                           int tid) {
  const int lane = tid & 63, wv = tid >> 6, wr = wv >> 2, wt = wv & 3;
  const int wv_u = __builtin_amdgcn_readfirstlane(wv);
  const int nsteps = a.K / kTK;
#pragma unroll
  for (int i = 0; i < kBI; ++i)
#pragma unroll
    for (int j = 0; j < kBJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  TiledCodes codes;
  TiledIds ids;
  // step 0 into buffer 0; the hash ids of step 1 in registers
  if constexpr (FUSED) issue_ids(ids, a, m0, 0, tid);
  issue_step<FUSED>(codes, ids, a, lds, m0, n0, 0, nsteps > 1 ? kTK : 0, wv_u, lane, tid);
  if constexpr (FUSED) store_codes(codes, lds + kOp, tid);
  stage_barrier();
  // step k: loads of step k + 1 into the other buffer (read during step k - 1, which every
  // wave has finished at the barrier), the hash ids of step k + 2, then the MFMAs of step k
  // The loop has no branches around loads (a load under a branch makes the compiler wait for
  // it at the join): in the last step the loads repeat that step into the free buffer.
  for (int k = 0; k < nsteps; ++k) {
    char* cur = lds + (k & 1) * kStage;
    char* nxt = lds + ((k + 1) & 1) * kStage;
    const int k1 = k + 1 < nsteps ? k + 1 : k;
    const int k2 = k + 2 < nsteps ? k + 2 : k1;
    issue_step<FUSED>(codes, ids, a, nxt, m0, n0, k1 * kTK, k2 * kTK, wv_u, lane, tid);
    asm volatile("" ::: "memory");
    stage_mma(acc, cur, lane, wr, wt);
    if constexpr (FUSED) store_codes(codes, nxt + kOp, tid);
    stage_barrier();
  }
}

__device__ __forceinline__ uint32_t* tcounter(const TiledArgs& a, int64_t tb, int s) {
  return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(a.ws) + 256 + (size_t(tb) * 4 + s) * 256);
}
// gate slots: [token block][value column block][stream][256 tokens] words
__device__ __forceinline__ uint32_t* tslot(const TiledArgs& a, int64_t tb, int vcb, int s) {
  return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(a.ws) + a.slot_off) +
         ((size_t(tb) * a.n_vcb + vcb) * 4 + s) * kTM;
}
// partial sums: [token block][stream][column block within the stream][256 tokens][3]
__device__ __forceinline__ float* tpartial(const TiledArgs& a, int64_t tb, int s, int cbs) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + a.part_off) +
         ((size_t(tb) * 4 + s) * a.n_vcb + cbs) * (kTM * 3);
}

// Hash ids of the tile's tokens that name no table row (each (token, column) pair counts 1).
__device__ __forceinline__ void count_bad_ids(const TiledArgs& a, int64_t m0, int tid) {
  if (a.err_count == nullptr) return;
  const int64_t m1 = m0 + kTM < a.M ? m0 + kTM : a.M;
  const int64_t n = (m1 - m0) * a.n_cols;
  const int64_t* ids = a.hash_ids + m0 * a.n_cols;
  int bad = 0;
  for (int64_t e = tid; e < n; e += kThreads) {
    const int64_t r = ids[e];
    bad += (r < 0 || r >= a.n_rows) ? 1 : 0;
  }
  if (bad) atomicAdd(a.err_count, bad);
}

// Key tile epilogue: this tile's share of the gate's three per-token sums (|h|^2, |k|^2 and
// the weighted dot product over the tile's 256 features of stream s), posted to the workspace;
// the last of the stream's key tiles evaluates the 256 gates and hands them to the value tiles.
__device__ __forceinline__ void key_epilogue(const TileAcc& acc, const TiledArgs& a, char* lds, int* s_last,
                                             int64_t tb, int64_t m0, int s, int cbs, int d0, int tid) {
  const int lane = tid & 63, wv = tid >> 6, wr = wv >> 2, wt = wv & 3;
  float (*red)[kTM][3] = reinterpret_cast<float (*)[kTM][3]>(lds);  // [2 column halves][256][3]
  float pa[kBJ], pk[kBJ], pd[kBJ];
#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    const int64_t m = m0 + 64 * wt + 16 * j + (lane & 15);
    const int64_t mm = m < a.M ? m : a.M - 1;
    float sa = 0.f, sk = 0.f, sd = 0.f;
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
      const int d = d0 + 16 * i + 4 * (lane >> 4);
      const u32x2 xw = *reinterpret_cast<const u32x2*>(a.x + (mm * 4 + s) * a.dim + d);
      const f32x4 q4 = *reinterpret_cast<const f32x4*>(a.q_weight + s * a.dim + d);
      const f32x4 k4 = *reinterpret_cast<const f32x4*>(a.k_weight + s * a.dim + d);
      const float h[4] = {bf16_lo(xw.x), bf16_hi(xw.x), bf16_lo(xw.y), bf16_hi(xw.y)};
      const float key[4] = {bf16_round(acc[i][j].x), bf16_round(acc[i][j].y), bf16_round(acc[i][j].z),
                            bf16_round(acc[i][j].w)};
      const float wq[4] = {q4.x * k4.x, q4.y * k4.y, q4.z * k4.z, q4.w * k4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sa += h[r] * h[r];
        sk += key[r] * key[r];
        sd += (h[r] * wq[r]) * key[r];
      }
    }
    sa += __shfl_xor(sa, 16, 64);
    sa += __shfl_xor(sa, 32, 64);
    sk += __shfl_xor(sk, 16, 64);
    sk += __shfl_xor(sk, 32, 64);
    sd += __shfl_xor(sd, 16, 64);
    sd += __shfl_xor(sd, 32, 64);
    pa[j] = sa;
    pk[j] = sk;
    pd[j] = sd;
  }
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < kBJ; ++j) {
      const int t = 64 * wt + 16 * j + lane;
      red[wr][t][0] = pa[j];
      red[wr][t][1] = pk[j];
      red[wr][t][2] = pd[j];
    }
  }
  __syncthreads();
  if (tid < kTM) {
    float* P = tpartial(a, tb, s, cbs) + tid * 3;
    store_coherent(P + 0, red[0][tid][0] + red[1][tid][0]);
    store_coherent(P + 1, red[0][tid][1] + red[1][tid][1]);
    store_coherent(P + 2, red[0][tid][2] + red[1][tid][2]);
  }
  drain_memory_ops();
  __syncthreads();
  if (tid == 0) *s_last = (atomic_add_relaxed(tcounter(a, tb, s), 1u) == uint32_t(a.n_vcb - 1)) ? 1 : 0;
  __syncthreads();
  if (*s_last && tid < kTM) {
    // every column block of this stream has posted: sum in column-block order
    float A = 0.f, Kq = 0.f, D = 0.f;
    for (int base = 0; base < a.n_vcb; base += 8) {
      float v[8][3];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int c = base + q < a.n_vcb ? base + q : base;
        const float* P = tpartial(a, tb, s, c) + tid * 3;
        v[q][0] = load_coherent(P + 0);
        v[q][1] = load_coherent(P + 1);
        v[q][2] = load_coherent(P + 2);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (base + q < a.n_vcb) {
          A += v[q][0];
          Kq += v[q][1];
          D += v[q][2];
        }
      }
    }
    const float fd = float(a.dim);
    const float rstd = __frsqrt_rn(A / fd + a.eps) * __frsqrt_rn(Kq / fd + a.eps);
    const float dot = D * rstd * a.inv_sqrt_dim;
    const float z = copysignf(sqrtf(fmaxf(fabsf(dot), a.clamp)), dot);
    const float g = 1.0f / (1.0f + expf(-z));
    const int64_t m = m0 + tid;
    const bool open = m < a.M && (a.token_mask == nullptr || a.token_mask[m] != 0);
    // gates are >= 0: the sign bit marks a slot as written
    const uint32_t bits = __float_as_uint(open ? g : 0.0f) | 0x80000000u;
    if (tid == 0) store_relaxed(tcounter(a, tb, s), 0u);
    for (int v = 0; v < a.n_vcb; ++v) store_relaxed(tslot(a, tb, v, s) + tid, bits);
    // the partials are consumed: leave them zero, so that the whole workspace is zero again
    // after the call (any schedule may use it next)
    for (int c = 0; c < a.n_vcb; ++c) {
      float* P = tpartial(a, tb, s, c) + tid * 3;
      store_coherent(P + 0, 0.0f);
      store_coherent(P + 1, 0.0f);
      store_coherent(P + 2, 0.0f);
    }
  }
}

// Value tile epilogue: wait for the 4 x 256 gates of the token block, then
// out = h + gate * value on every stream for the tile's 256 features.
__device__ __forceinline__ void value_epilogue(const TileAcc& acc, const TiledArgs& a, char* lds, int64_t tb,
                                               int64_t m0, int cbs, int d0, int tid) {
  const int lane = tid & 63, wv = tid >> 6, wt = wv & 3;
  float (*gates)[kTM] = reinterpret_cast<float (*)[kTM]>(lds);  // [4 streams][256]
  // each thread waits for two slot words (stream w >> 8, token w & 255) and clears them
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int w = tid + kThreads * q;
    const int s2 = w >> 8, t = w & 255;
    uint32_t* slot = tslot(a, tb, cbs, s2) + t;
    uint32_t bits = 0u, it = 0;
    while ((bits = load_relaxed(slot)) == 0u) {
      __builtin_amdgcn_s_sleep(4);
      if (++it > a.spin_budget) {
        atomic_add_relaxed(reinterpret_cast<uint32_t*>(a.ws), 1u);
        break;
      }
    }
    store_relaxed(slot, 0u);
    gates[s2][t] = __uint_as_float(bits & 0x7FFFFFFFu);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    const int t = 64 * wt + 16 * j + (lane & 15);
    const int64_t m = m0 + t;
    if (m >= a.M) continue;
    const bool open = a.token_mask == nullptr || a.token_mask[m] != 0;
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
      const int d = d0 + 16 * i + 4 * (lane >> 4);
      const float v[4] = {bf16_round(acc[i][j].x), bf16_round(acc[i][j].y), bf16_round(acc[i][j].z),
                          bf16_round(acc[i][j].w)};
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const size_t off = size_t(m * 4 + s2) * a.dim + d;
        const u32x2 xw = *reinterpret_cast<const u32x2*>(a.x + off);
        const float g = gates[s2][t];
        u32x2 o = xw;
        if (open) {
          o.x = pack_bf16x2(bf16_lo(xw.x) + g * v[0], bf16_hi(xw.x) + g * v[1]);
          o.y = pack_bf16x2(bf16_lo(xw.y) + g * v[2], bf16_hi(xw.y) + g * v[3]);
        }
        if (open || a.out != a.x) *reinterpret_cast<u32x2*>(a.out + off) = o;
      }
    }
  }
}

template <bool FUSED>
__global__ __launch_bounds__(kThreads) void k_tiled(TiledArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wr = wv >> 2, wt = wv & 3;
  const int64_t n_tb = (a.M + kTM - 1) / kTM;
  const int64_t b = blockIdx.x;
  const int64_t tb = b % n_tb;
  const int cb = int(b / n_tb);
  const int64_t m0 = tb * kTM;
  const int n0 = cb * kTN;

  TileAcc acc;
  tiled_gemm<FUSED>(acc, a, lds, m0, n0, tid);
  // the last K step ended with a barrier: the stage buffers are free for the epilogue

  if constexpr (!FUSED) {
#pragma unroll
    for (int j = 0; j < kBJ; ++j) {
      const int64_t m = m0 + 64 * wt + 16 * j + (lane & 15);
      if (m < a.M) {
#pragma unroll
        for (int i = 0; i < kBI; ++i) {
          const int n = n0 + 128 * wr + 16 * i + 4 * (lane >> 4);
          *reinterpret_cast<u32x2*>(a.kv + m * a.N + n) =
              u32x2{pack_bf16x2(acc[i][j].x, acc[i][j].y), pack_bf16x2(acc[i][j].z, acc[i][j].w)};
        }
      }
    }
  } else {
    const int s = n0 / a.dim;  // a tile lies in one segment: dim is a multiple of 256
    const int cbs = (n0 - s * a.dim) / kTN;
    const int d0 = n0 - s * a.dim + 128 * wr;
    if (cb == 0) count_bad_ids(a, m0, tid);
    if (s < 4)
      key_epilogue(acc, a, lds, &s_last, tb, m0, s, cbs, d0, tid);
    else
      value_epilogue(acc, a, lds, tb, m0, cbs, d0, tid);
  }
}

hipError_t launch_tiled_impl(const TiledArgs& a, bool fused, hipStream_t stream) {
  const int64_t n_tb = (a.M + kTM - 1) / kTM;
  const int64_t tiles = n_tb * (a.N / kTN);
  if (tiles <= 0 || tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const void* fn = fused ? reinterpret_cast<const void*>(&k_tiled<true>)
                         : reinterpret_cast<const void*>(&k_tiled<false>);
  static bool attr_set[2] = {false, false};
  if (!attr_set[fused]) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    attr_set[fused] = true;
  }
  TiledArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(fn, dim3(unsigned(tiles)), dim3(kThreads), params, kLds, stream);
}

size_t tiled_layout(TiledArgs* a, int64_t M, int dim) {
  const int64_t n_tb = (M + kTM - 1) / kTM;
  const int n_vcb = dim / kTN;
  size_t off = 256 + size_t(n_tb) * 4 * 256;  // header, counters (one 256-byte line each)
  const size_t slot_off = off;
  off += size_t(n_tb) * n_vcb * 4 * kTM * 4;
  off = (off + 255) & ~size_t(255);
  const size_t part_off = off;
  off += size_t(n_tb) * 4 * n_vcb * kTM * 3 * 4;
  if (a != nullptr) {
    a->n_vcb = n_vcb;
    a->slot_off = slot_off;
    a->part_off = part_off;
  }
  return off;
}

}  // namespace

bool tiled_shape_ok(int N, int K, int dim, int head_dim, int scale_block, bool fused) {
  if (N % kTN != 0 || K % kTK != 0) return false;
  if (fused && (dim % kTN != 0 || head_dim % kTK != 0 || scale_block % 16 != 0)) return false;
  return true;
}

size_t tiled_workspace_bytes(int64_t M, int dim) { return tiled_layout(nullptr, M, dim); }

hipError_t launch_kv_proj_tiled(const TiledArgs& a, hipStream_t stream) { return launch_tiled_impl(a, false, stream); }

hipError_t launch_forward_tiled(TiledArgs a, void* workspace, hipStream_t stream) {
  a.ws = workspace;
  tiled_layout(&a, a.M, a.dim);
  return launch_tiled_impl(a, true, stream);
}

}  // namespace engram
