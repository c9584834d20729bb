// Weight-streaming wkv projection for small token counts (decode), alone or fused with the
// row gather, the per-stream gate and the residual add.
//
// Schedule.  The N = (hc + 1) * dim output columns are the rows of the wkv matrix ([N, K], K
// contiguous).  A persistent grid of G workgroups (one per CU) gives workgroup w the contiguous
// rows [4 floor(w Q / G), 4 floor((w + 1) Q / G)) with Q = N / 4, so every byte of wkv is read
// exactly once per 64-token block and the load is balanced to within four rows (25600 rows on
// 256 CUs: exactly 100 each).  A workgroup's rows form 16-row blocks starting at its first row;
// rows of a last, partial block past the workgroup's end are neither loaded from HBM (their
// loads repeat the last row) nor written.
// The four waves of a workgroup split K into four contiguous quarters; each wave multiplies its
// quarter of the workgroup's rows against its quarter of the 64 token rows, and the four
// K-partials are summed in a fixed order through LDS at the end.
//
// Two K loops feed the same reduction and epilogue:
//  * wide (each K quarter a multiple of 128 features, head_dim a multiple of 128): weights are
//    copied global -> LDS (global_load_lds_dwordx4) 4 rows x 256 contiguous bytes per wave
//    instruction -- HBM streams at close to its peak only with runs of this length -- into a
//    wave-private slot per row block, with the 16-byte chunks of each row permuted so that the
//    MFMA fragment reads hit distinct banks.  A whole chunk (all row blocks x 128 features) of
//    copies stays in flight without holding registers; the row-block count is a template
//    constant so no load sits behind a branch.
//  * narrow (any shape the library accepts): fragments are loaded in MFMA layout directly
//    (16 rows x 64 bytes per instruction) with a ring of U steps in flight.
//  * wide with MXFP8 weights (e4m3fn codes, one E8M0 scale per 32 features of a row): the
//    same schedule over half the bytes.  A row block's slot holds 16 rows x 128 bytes of codes
//    (8 rows x 128 bytes per copy instruction: 128-byte runs stream as fast as 256-byte ones when
//    the rows are 6 KB apart) and the chunk's scale dword of each row.  With a table of fp32
//    scales the fragments are dequantised to bf16 in registers, exactly (a power-of-two scale),
//    and meet the same bf16 MFMA.  With an MXFP8 table both operands stay fp8 codes and one
//    scaled fp8 MFMA (16 x 16 x 128, E8M0 scales per 32 features on both sides) takes a whole
//    chunk: a quarter of the MFMA instructions and no dequantisation at all.
// In the fused kernel the token operand is gathered: each lane loads the 8 fp8 codes and the
// scale it needs straight from the table rows named by the hash ids (staged once per token
// block in LDS) and dequantises them in registers, one chunk ahead of use.
//
// MFMA roles: the weight rows are the A operand (16 rows), the tokens the B operand (16 tokens),
// so every lane ends up holding four consecutive output columns of one token.
//
// Fused epilogue.  Key columns of stream s contribute, per token, partial sums of h^2, key^2
// and h * q * k * key over their features; each workgroup posts one partial per (token,
// stream) and bumps a per-stream counter.  The workgroup that arrives last for a stream sums
// the partials of all contributing workgroups in workgroup order (deterministic), evaluates
// the gate of the 64 tokens and writes it into the slots of the workgroups that apply it.  With
// one token block (decode), value workgroups leave their bf16 values in tiles and exit, and
// apply workgroups (ids after the streaming ones) wait for a tile and its gates, then write
// out = bf16(h + g * value) for the tile's features on all four streams; over several token
// blocks, the value workgroups themselves wait for their slots and write out.
// Only workgroups of higher ids wait, on work of lower ids that never waits (value columns
// belong to the highest streaming ids, apply workgroups come after them).  Workgroups are
// dispatched in id order and at most one runs per CU, so every workgroup that one waits on is
// running or done before the wait starts; each wait is bounded as well, and a time-out is
// recorded in the workspace header instead of hanging.  Partial sums, tiles and gates pass
// between workgroups through device-coherent loads and stores ordered by store completion and
// barriers; counters, slots and tiles are reset by their last user, so a call leaves them zero.
#include <string.h>

#include <mutex>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace engram {

namespace {

constexpr int kTB = 64;                          // tokens per token block
constexpr int kRedBytes = 4 * 2 * 4 * 64 * 16;   // K-partial reduction buffer (two row blocks)
constexpr int kWBlk = 16 * 256;                  // LDS slot of one row block x 128 features
constexpr int kWBlk8 = 16 * 128;                 // the same with MXFP8 weights (codes)
constexpr int kTokBuf_ = 9 * 1024;               // fused wide loop: token buffer per wave
// LDS in front of the staged hash ids: the weight slots of the wide loop (4 waves x nblk row
// blocks) and the token buffers, which the one-round K-partial reduction (nblk x 16 KB) reuses
// afterwards.
__host__ __device__ constexpr int wide_lds_bytes(int nblk, bool fused, bool w8) {
  return (4 * nblk * (w8 ? kWBlk8 : kWBlk) + (fused ? 4 * kTokBuf_ : 0)) > (nblk * 16384 > kRedBytes ? nblk * 16384 : kRedBytes)
             ? 4 * nblk * (w8 ? kWBlk8 : kWBlk) + (fused ? 4 * kTokBuf_ : 0)
             : (nblk * 16384 > kRedBytes ? nblk * 16384 : kRedBytes);
}

// First row of workgroup w (rows are dealt in groups of four: Q = N / 4 groups).
// (32-bit arithmetic: the host keeps G * Q below 2^32.)
__device__ __forceinline__ int row_begin(int w, int Q, int G) { return 4 * int(uint32_t(w) * uint32_t(Q) / uint32_t(G)); }
// workgroup that owns a row
__device__ __forceinline__ int owner_of_row(int row, int Q, int G) {
  return int((uint32_t(row / 4 + 1) * uint32_t(G) - 1u) / uint32_t(Q));
}

// The rows of one workgroup: [r0, r1) in nblk blocks of 16 (the last one possibly partial).
struct Rows {
  int r0, r1, nblk;
};
__device__ __forceinline__ Rows rows_of(int w, int N, int G) {
  Rows r;
  r.r0 = row_begin(w, N / 4, G);
  r.r1 = row_begin(w + 1, N / 4, G);
  r.nblk = (r.r1 - r.r0 + 15) / 16;
  return r;
}

// Eight fp8 codes (two dwords) times one fp32 scale -> eight bf16 (an MFMA operand).  NaN
// payloads are not canonicalised here: a NaN operand makes the products NaN either way.
__device__ __forceinline__ u32x4 dequant8(u32x2 c, float s) {
  const u32x2 lo = dequant4_raw(c.x, s), hi = dequant4_raw(c.y, s);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

__device__ __forceinline__ u32x4 masked(u32x4 v, uint32_t k) { return u32x4{v.x & k, v.y & k, v.z & k, v.w & k}; }

// Token fragment source of one lane for one 32-feature step: gathered codes + scale, or a row
// slice of emb, and an all-ones / zero mask for rows that must read as zeros.
struct TokFrag {
  u32x2 code;
  float scale;
  u32x4 emb;
  uint32_t keep;
};

// Loads the token fragment of sub-block t for features [f, f + 8) of this lane (branch-free:
// invalid ids read row 0 and out-of-range tokens read the last token, both masked at use).
template <bool FUSED>
__device__ __forceinline__ void load_tok(TokFrag& tf, const StreamArgs& a, const int64_t* s_ids, int64_t m0,
                                         int t, int f, int lane) {
  if constexpr (FUSED) {
    const int j = f / a.head_dim;
    const int cc = f - j * a.head_dim;
    const int64_t r = s_ids[(16 * t + (lane & 15)) * a.n_cols + j];
    const int64_t rr = r >= 0 ? r : 0;
    tf.keep = r >= 0 ? 0xFFFFFFFFu : 0u;
    tf.code = *reinterpret_cast<const u32x2*>(a.table + rr * a.head_dim + cc);
    tf.scale = load_scale(a.scales, rr * (a.head_dim / a.scale_block) + cc / a.scale_block, a.scale_e8m0);
  } else {
    const int64_t m = m0 + 16 * t + (lane & 15);
    tf.keep = m < a.M ? 0xFFFFFFFFu : 0u;
    const int64_t mm = m < a.M ? m : a.M - 1;
    tf.emb = *reinterpret_cast<const u32x4*>(a.emb + mm * a.K + f);
  }
}

template <bool FUSED>
__device__ __forceinline__ u32x4 tok_operand(const TokFrag& tf) {
  if constexpr (FUSED) return masked(dequant8(tf.code, tf.scale), tf.keep);
  else return masked(tf.emb, tf.keep);
}

// ------------------------------------------------------------------------------ narrow K loop
template <int NRB, int U, bool FUSED>
struct NarrowSlot {
  u32x4 w[NRB];
  TokFrag tok[4];
};

template <int NRB, int U, bool FUSED>
__device__ __forceinline__ void narrow_issue(NarrowSlot<NRB, U, FUSED>& sl, const StreamArgs& a, const int64_t* s_ids,
                                             int64_t m0, const Rows& rw, int step, int lane, int wv) {
  const int f = wv * (a.K >> 2) + 32 * step + 8 * (lane >> 4);  // first of this lane's 8 features
#pragma unroll
  for (int i = 0; i < NRB; ++i) {
    int row = rw.r0 + 16 * i + (lane & 15);
    row = row < rw.r1 ? row : rw.r1 - 1;  // past the workgroup's rows: re-read (cache hit)
    sl.w[i] = *reinterpret_cast<const u32x4*>(a.wkv + size_t(row) * a.K + f);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) load_tok<FUSED>(sl.tok[t], a, s_ids, m0, t, f, lane);
}

template <int NRB, int U, bool FUSED>
__device__ __forceinline__ void narrow_loop(f32x4 (&acc)[NRB][4], const StreamArgs& a, const int64_t* s_ids,
                                            int64_t m0, const Rows& rw, int lane, int wv) {
  const int nstep = (a.K >> 2) / 32;  // 32-feature steps per wave; a multiple of U
  NarrowSlot<NRB, U, FUSED> ring[U];
#pragma unroll
  for (int p = 0; p < U; ++p) {
    narrow_issue<NRB, U, FUSED>(ring[p], a, s_ids, m0, rw, p, lane, wv);
    // pin the issue order: the compiler otherwise sinks ring loads into the next iteration
    asm volatile("" ::: "memory");
  }
  for (int c0 = 0; c0 < nstep; c0 += U) {
#pragma unroll
    for (int p = 0; p < U; ++p) {
      u32x4 bt[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) bt[t] = tok_operand<FUSED>(ring[p].tok[t]);
#pragma unroll
      for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = mfma16x16x32(ring[p].w[i], bt[t], acc[i][t]);
      const int nxt = c0 + p + U < nstep ? c0 + p + U : nstep - 1;
      narrow_issue<NRB, U, FUSED>(ring[p], a, s_ids, m0, rw, nxt, lane, wv);
      asm volatile("" ::: "memory");
    }
  }
}

// ------------------------------------------------------------------------------ wide K loop
// Chunk c of a wave covers features [q0 + 128 c', q0 + 128 c' + 128) of its quarter q0, with
// c' = (c + 5 w) mod (chunks per quarter) for workgroup w (see wide_loop).  Weight
// unit (row block i, chunk c): copy instruction k in 0..3 fills LDS bytes [1024 k, 1024 k + 1024)
// of the row block's slot, lane l at 16 l: row 4 k + l / 16 of the block, position l % 16, which
// holds the 16-byte chunk (l % 16) ^ row -- four rows of 256 contiguous bytes from HBM.  Each
// lane then reads, for step s in 0..3, row l % 16 at features 32 (l / 16) + 8 s (chunk
// 4 (l / 16) + s, at position chunk ^ row): the pairing of A and B rows along K is free, and
// this order gives every lane 32 contiguous token features per chunk (two 16-byte code loads
// and one scale in the fused kernel).
//
// When `live` is false (the refill after the last chunk) the same instructions read the first
// 256 bytes of rows 0..15 instead: a 4 KB cache-resident region, so no extra HBM traffic.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void wide_copy_w(char* slot, const StreamArgs& a, const Rows& rw, int i, int f_chunk,
                                            bool live, int lane) {
  const int rbase = live ? rw.r0 + 16 * i : 0;
  const int rlast = live ? rw.r1 - 1 : 15;
  const size_t fbase = live ? size_t(f_chunk) : 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = 4 * k + (lane >> 4);
    const int r = rbase + rr;
    const size_t row = size_t(r < rlast ? r : rlast);
    const int chunk = (lane & 15) ^ rr;
    // cache policy 2: non-temporal (each weight byte is read once)
    __builtin_amdgcn_global_load_lds((const void*)(a.wkv + row * a.K + fbase + 8 * chunk),
                                     (lds_ptr_t)(slot + k * 1024), 16, 0, 2);
  }
}

// MXFP8 weights, unit (row block i, chunk c): copy k in 0..1 fills slot bytes [1024 k, 1024 k +
// 1024), lane l at 16 l: row 8 k + l / 8, position l % 8, which holds the 16-byte part
// (l % 8) ^ ((row >> 1) & 7) of the row's 128 chunk bytes (rows 128 bytes apart: with this
// permutation the 16 rows of a fragment read cover all banks).  Not live: the first 128 bytes of
// rows 0..15 (cache resident).  The E8M0 scales of the workgroup's rows are not copied per
// chunk: the whole table of its rows sits in LDS (load_scale_table), because one 4-byte read per
// row and chunk, rows K / 32 bytes apart, cost ~6 us of the decode call.
__device__ __forceinline__ void wide_copy_w8(char* slot, const StreamArgs& a, const Rows& rw, int i, int f_chunk,
                                             bool live, int lane) {
  const int rbase = live ? rw.r0 + 16 * i : 0;
  const int rlast = live ? rw.r1 - 1 : 15;
  const size_t fbase = live ? size_t(f_chunk) : 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int rr = 8 * k + (lane >> 3);
    const int r = rbase + rr;
    const size_t row = size_t(r < rlast ? r : rlast);
    const int part = (lane & 7) ^ ((rr >> 1) & 7);
    __builtin_amdgcn_global_load_lds((const void*)(a.wkv8 + row * a.K + fbase + 16 * part),
                                     (lds_ptr_t)(slot + k * 1024), 16, 0, 2);
  }
}

// The E8M0 scales of rows [r0, r1): one contiguous run of (r1 - r0) K / 32 bytes (a multiple of
// 16, at a 16-byte aligned offset: r0 is a multiple of 4 and K of 128), copied 16 bytes per lane
// by the workgroup's 256 threads.  Not waited for here.
__device__ __forceinline__ void load_scale_table(char* table, const StreamArgs& a, const Rows& rw, int tid) {
  const int n16 = (rw.r1 - rw.r0) * (a.K / 32) / 16;
  const char* src = reinterpret_cast<const char*>(a.wkv8s) + size_t(rw.r0) * (a.K / 32);
  const int wv = tid >> 6, lane = tid & 63;
  for (int base = 64 * wv; base < n16; base += 256) {
    if (base + lane < n16)
      __builtin_amdgcn_global_load_lds((const void*)(src + 16 * size_t(base + lane)), (lds_ptr_t)(table + 16 * base),
                                       16, 0, 0);
  }
}

// The scale dword of the lane's row (l % 16 of row block i, the last row for rows past the
// workgroup's end) at features [f, f + 128).
__device__ __forceinline__ uint32_t table_scales(const char* table, const StreamArgs& a, const Rows& rw, int i,
                                                 int f_chunk, int lane) {
  const int r = 16 * i + (lane & 15);
  const int rl = rw.r1 - rw.r0 - 1;
  return *reinterpret_cast<const uint32_t*>(table + (r < rl ? r : rl) * (a.K / 32) + f_chunk / 32);
}

// Raw MXFP8 fragment of one lane: codes of its row (l % 16) at features 32 (l / 16) + [0, 32)
// (parts 2 (l / 16) and 2 (l / 16) + 1) and the scale dword.
struct Frag8 {
  u32x4 c0, c1;
  uint32_t sdw;
};
__device__ __forceinline__ Frag8 wide_read_w8(const char* slot, uint32_t sdw, int lane) {
  const int rr = lane & 15, p0 = 2 * (lane >> 4), sw = (rr >> 1) & 7;
  Frag8 f;
  f.c0 = *reinterpret_cast<const u32x4*>(slot + rr * 128 + 16 * (p0 ^ sw));
  f.c1 = *reinterpret_cast<const u32x4*>(slot + rr * 128 + 16 * ((p0 + 1) ^ sw));
  f.sdw = sdw;
  return f;
}
// Raw fragment in the scaled fp8 MFMA's layout: row l % 16 at chunk features 16 (l / 16) +
// [0, 16) and 64 + 16 (l / 16) + [0, 16) (parts l / 16 and l / 16 + 4), and the scale dword
// (the MFMA takes the scale of features 32 (l / 16) .. from this lane: byte l / 16).
__device__ __forceinline__ Frag8 wide_read_w8_mx(const char* slot, uint32_t sdw, int lane) {
  const int rr = lane & 15, g = lane >> 4, sw = (rr >> 1) & 7;
  Frag8 f;
  f.c0 = *reinterpret_cast<const u32x4*>(slot + rr * 128 + 16 * (g ^ sw));
  f.c1 = *reinterpret_cast<const u32x4*>(slot + rr * 128 + 16 * ((g + 4) ^ sw));
  f.sdw = sdw;
  return f;
}

// The four bf16 operands (steps s = 0..3: features 8 s .. 8 s + 7 of the lane's 32); the
// lane's 32 features share the scale in byte l / 16 of the dword.
// (v_cvt_scalef32_pk_bf16_fp8: two codes times the scale to two bf16 in one instruction; the
// product of an fp8 value and a power of two is a bf16 number wherever it is not subnormal.)
template <bool HI>
__device__ __forceinline__ uint32_t cvt2_scaled(uint32_t c, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, sc, HI));
}
__device__ __forceinline__ u32x4 dequant8_scaled(uint32_t c0, uint32_t c1, float sc) {
  return u32x4{cvt2_scaled<false>(c0, sc), cvt2_scaled<true>(c0, sc), cvt2_scaled<false>(c1, sc),
               cvt2_scaled<true>(c1, sc)};
}
__device__ __forceinline__ void wide_operands_w8(u32x4 (&wf)[4], const Frag8& f, int lane) {
  const float sc = e8m0_to_f32((f.sdw >> (8 * (lane >> 4))) & 0xFFu);
  wf[0] = dequant8_scaled(f.c0.x, f.c0.y, sc);
  wf[1] = dequant8_scaled(f.c0.z, f.c0.w, sc);
  wf[2] = dequant8_scaled(f.c1.x, f.c1.y, sc);
  wf[3] = dequant8_scaled(f.c1.z, f.c1.w, sc);
}

// Dense token operands (the projection alone) of one chunk for one lane: sub-block t, features
// f_chunk + 32 * (lane / 16) + [0, 32) of emb, four dwordx4 per sub-block, loaded into
// registers one chunk ahead.  (The fused kernel copies gathered codes into LDS instead.)
struct WideTok {
  u32x4 v[4][4];
  uint32_t keep[4];
};

__device__ __forceinline__ void wide_issue_tok(WideTok& tk, const StreamArgs& a, int64_t m0, int f_chunk,
                                               int lane) {
  const int f = f_chunk + 32 * (lane >> 4);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t m = m0 + 16 * t + (lane & 15);
    tk.keep[t] = m < a.M ? 0xFFFFFFFFu : 0u;
    const int64_t mm = m < a.M ? m : a.M - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(a.emb + mm * a.K + f);
#pragma unroll
    for (int q = 0; q < 4; ++q) tk.v[t][q] = src[q];
  }
}

// Operand of step s (features 8 s .. 8 s + 7 of the lane's 32) for sub-block t.
__device__ __forceinline__ u32x4 wide_operand(const WideTok& tk, int t, int s) { return masked(tk.v[t][s], tk.keep[t]); }

// Fused kernel: the gathered token codes and scales of one chunk are copied global -> LDS as
// well, into a wave-private 9 KB buffer, so that the K loop holds no register loads: the
// compiler would otherwise wait for every copy in flight before each use of a token register.
// Codes: the chunk's 128 features are one 128-byte piece of each token's table row (a chunk
// stays inside one column), and copy k (0..7) fills buffer bytes [1024 k, 1024 k + 1024) with
// the pieces of tokens 8 k .. 8 k + 7, eight lanes per token, so every cache line the gather
// touches is read whole.  Row `tok` of the buffer keeps its 16-byte part p at position
// p ^ ((tok >> 1) & 7), which spreads the reads of 16 consecutive tokens over all banks.
// Scales: copy 8 + t puts the scale a lane needs for sub-block t (token 16 t + lane % 16,
// features 32 (lane / 16) ..) at 8192 + 256 t + 4 lane: the fp32 scale, or for E8M0 scales the
// aligned dword that holds the byte (a row's E8M0 scales are whole dwords: the layout check
// asks for a multiple of 4 per row), which the read takes apart.  `keep` marks lanes whose
// hash id names a table row.
constexpr int kTokBuf = kTokBuf_;

template <bool SCALES = true, typename IdT = int64_t>
__device__ __forceinline__ void wide_copy_tok(char* tbuf, uint32_t (&keep)[4], const StreamArgs& a,
                                              const IdT* s_ids, int f_chunk, int lane) {
  const int j = f_chunk / a.head_dim;
  const int cc0 = f_chunk - j * a.head_dim;
  const int nb = a.head_dim / a.scale_block;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int tok = 8 * k + (lane >> 3);
    const int64_t r = s_ids[tok * a.n_cols + j];
    const int64_t rr = r >= 0 ? r : 0;
    const int part = (lane & 7) ^ ((tok >> 1) & 7);
    __builtin_amdgcn_global_load_lds((const void*)(a.table + rr * a.head_dim + cc0 + 16 * part),
                                     (lds_ptr_t)(tbuf + k * 1024), 16, 0, 0);
  }
  const int cc = cc0 + 32 * (lane >> 4);
  const int sbyte = a.scale_e8m0 ? 1 : 4;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t r = s_ids[(16 * t + (lane & 15)) * a.n_cols + j];
    const int64_t rr = r >= 0 ? r : 0;
    keep[t] = r >= 0 ? 0xFFFFFFFFu : 0u;
    if constexpr (SCALES) {
      const size_t off = size_t(rr * nb + cc / a.scale_block) * sbyte;
      __builtin_amdgcn_global_load_lds((const void*)(static_cast<const char*>(a.scales) + (off & ~size_t(3))),
                                       (lds_ptr_t)(tbuf + 8192 + t * 256), 4, 0, 0);
    }
  }
}

// Scaled fp8 MFMA (E8M0 table): the E8M0 scales of the gathered rows of this wave's columns,
// gathered once per token block into a wave-private table instead of one dword per token and
// chunk with the codes.  The wave's K quarter covers whole columns j0 .. j0 + ncw - 1 (the host
// asks K / 4 to be a multiple of head_dim); entry (token, jj) holds the row's head_dim /
// scale_block bytes (whole dwords).  Not waited for here: the K loop's first waits cover them
// (issued earlier, they complete earlier).
__device__ __forceinline__ int tok_table_bytes(const StreamArgs& a) {
  return kTB * ((a.K >> 2) / a.head_dim) * (a.head_dim / a.scale_block);
}
__device__ __forceinline__ void load_tok_scales(char* tab, const StreamArgs& a, const int64_t* s_ids, int q0,
                                                int lane) {
  const int ncw = (a.K >> 2) / a.head_dim, nb = a.head_dim / a.scale_block, nd = nb >> 2;
  const int j0 = q0 / a.head_dim;
  const int n = kTB * ncw * nd;
  for (int base = 0; base < n; base += 64) {
    const int e = base + lane;
    if (e < n) {
      const int tok = e / (ncw * nd), jj = (e / nd) % ncw, d = e % nd;
      const int64_t r = s_ids[tok * a.n_cols + j0 + jj];
      const int64_t rr = r >= 0 ? r : 0;
      __builtin_amdgcn_global_load_lds((const void*)(static_cast<const char*>(a.scales) + rr * nb + 4 * d),
                                       (lds_ptr_t)(tab + 4 * base), 4, 0, 0);
    }
  }
}

// The 16 token operands of one chunk (steps s = 0..3 x sub-blocks t = 0..3) from the buffer:
// the lane's 32 features are the 16-byte parts 2 (lane / 16) and 2 (lane / 16) + 1 of its token.
// e8m0_shift: 0 for fp32 scales, else 8 x (byte offset of the lane's E8M0 scale in its dword).
__device__ __forceinline__ void wide_tok_operands(u32x4 (&bt)[4][4], const char* tbuf, const uint32_t (&keep)[4],
                                                  int lane, int e8m0, uint32_t e8m0_shift) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int tok = 16 * t + (lane & 15);
    const int sw = (tok >> 1) & 7;
    const int p0 = 2 * (lane >> 4);
    const u32x4 c0 = *reinterpret_cast<const u32x4*>(tbuf + tok * 128 + 16 * (p0 ^ sw));
    const u32x4 c1 = *reinterpret_cast<const u32x4*>(tbuf + tok * 128 + 16 * ((p0 + 1) ^ sw));
    const uint32_t sw32 = *reinterpret_cast<const uint32_t*>(tbuf + 8192 + t * 256 + 4 * lane);
    const float sc = e8m0 ? e8m0_to_f32((sw32 >> e8m0_shift) & 0xFFu) : __uint_as_float(sw32);
    bt[0][t] = masked(dequant8(u32x2{c0.x, c0.y}, sc), keep[t]);
    bt[1][t] = masked(dequant8(u32x2{c0.z, c0.w}, sc), keep[t]);
    bt[2][t] = masked(dequant8(u32x2{c1.x, c1.y}, sc), keep[t]);
    bt[3][t] = masked(dequant8(u32x2{c1.z, c1.w}, sc), keep[t]);
  }
}

// Token operands of one chunk for the scaled fp8 MFMA (MXFP8 table): sub-block t, token
// 16 t + lane % 16, parts lane / 16 and lane / 16 + 4 of its 128 chunk bytes as raw codes, and
// its E8M0 scale of features 32 (lane / 16) ..  Rows that read as zeros get zero codes and scale
// 2^0 (a NaN scale of the substitute row must not reach the sum).
// `ts` points at the lane's scale dword of token 0 in the wave's scale table (token stride
// `tstride` bytes).
__device__ __forceinline__ void wide_tok_operands_mx(u32x4 (&lo)[4], u32x4 (&hi)[4], int (&sc)[4], const char* tbuf,
                                                     const uint32_t (&keep)[4], int lane, const char* ts,
                                                     int tstride, uint32_t e8m0_shift) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int tok = 16 * t + (lane & 15);
    const int sw = (tok >> 1) & 7;
    const int g = lane >> 4;
    lo[t] = masked(*reinterpret_cast<const u32x4*>(tbuf + tok * 128 + 16 * (g ^ sw)), keep[t]);
    hi[t] = masked(*reinterpret_cast<const u32x4*>(tbuf + tok * 128 + 16 * ((g + 4) ^ sw)), keep[t]);
    const uint32_t sw32 = *reinterpret_cast<const uint32_t*>(ts + tok * tstride);
    sc[t] = keep[t] ? int((sw32 >> e8m0_shift) & 0xFFu) : 127;
  }
}

// Vector memory instructions of one chunk's token operands of a lane (fused: copies).
template <bool FUSED, bool MX = false>
constexpr int kTokLoads = MX ? 8 : (FUSED ? 12 : 16);

template <int NRB, bool FUSED, bool W8, bool MX>
__device__ __forceinline__ void wide_loop(f32x4 (&acc)[NRB][4], const StreamArgs& a, const int64_t* s_ids,
                                          char* slots, const char* stable, const char* ttable, int64_t m0,
                                          const Rows& rw, int lane, int wv) {
  constexpr int kSlot = W8 ? kWBlk8 : kWBlk;
  constexpr int kWIns = W8 ? 2 : 4;  // copy instructions per row block and chunk
  const int q0 = wv * (a.K >> 2);
  const int nch = (a.K >> 2) / 128;
  // Each workgroup walks its quarter's chunks starting at its own chunk (5 w mod nch), so that
  // the workgroups' copies in flight spread over many column offsets of the weight rows instead
  // of all sitting at the same one (a streaming probe of this pattern: 6.25 -> 6.59 TB/s).
  const int rot = int((5u * blockIdx.x) % uint32_t(nch));
  auto feat = [&](int c) { return q0 + 128 * ((c + rot) % nch); };
  char* my_slots = slots + wv * NRB * kSlot;
  char* my_tok = slots + 4 * NRB * kSlot + wv * kTokBuf;  // fused only
  WideTok tk;              // dense only
  uint32_t keep[4];        // fused only
  // prologue in the loop's issue order (tokens, then row blocks)
  if constexpr (FUSED) wide_copy_tok<!MX>(my_tok, keep, a, s_ids, feat(0), lane);
  else wide_issue_tok(tk, a, m0, feat(0), lane);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < NRB; ++i) {
    if constexpr (W8) wide_copy_w8(my_slots + i * kSlot, a, rw, i, feat(0), true, lane);
    else wide_copy_w(my_slots + i * kSlot, a, rw, i, feat(0), true, lane);
    asm volatile("" ::: "memory");
  }
  // Issue order per chunk c: the tokens of chunk c + 1, then (as row block i of chunk c is read)
  // the copies of row block i of chunk c + 1.  So when row block i of chunk c is read, the
  // copies of blocks i + 1 .. NRB - 1 of chunk c, the tokens of chunk c + 1 and the copies of
  // blocks 0 .. i - 1 of chunk c + 1 -- always kWIns (NRB - 1) + kTokLoads instructions -- may
  // still be in flight.
  constexpr int kInFlight = kWIns * (NRB - 1) + kTokLoads<FUSED, MX>;
  static_assert(kInFlight <= 63, "vmcnt range");
  const int fl = (lane & 15) * 256;  // this lane's fragment row in a slot
  for (int c = 0; c < nch; ++c) {
    const bool live = c + 1 < nch;
    const int fc = feat(c);                        // this chunk's first feature
    const int fn = feat(live ? c + 1 : c);         // next chunk (tokens re-read the last one)
    u32x4 bt[4][4];
    u32x4 bx_lo[4], bx_hi[4];  // MX: raw token codes and scales
    int bx_sc[4];
    if constexpr (FUSED) {
      // the token copies of chunk c have landed once only the weight copies of chunk c remain
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWIns * NRB) : "memory");
      // the lane's E8M0 scale byte within its dword (row scales are whole dwords)
      const int cc_cur = fc % a.head_dim + 32 * (lane >> 4);
      const uint32_t e8m0_shift = uint32_t((cc_cur / a.scale_block) & 3) * 8u;
      if constexpr (MX) {
        // the lane's dword in the wave's scale table: column jj of the quarter, block cc_cur / sb
        const int nb = a.head_dim / a.scale_block;
        const int jj = fc / a.head_dim - q0 / a.head_dim;
        const int tstride = ((a.K >> 2) / a.head_dim) * nb;
        const char* ts = ttable + jj * nb + ((cc_cur / a.scale_block) & ~3);
        wide_tok_operands_mx(bx_lo, bx_hi, bx_sc, my_tok, keep, lane, ts, tstride, e8m0_shift);
      } else {
        wide_tok_operands(bt, my_tok, keep, lane, a.scale_e8m0, e8m0_shift);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the buffer is read before its refill
      wide_copy_tok<!MX>(my_tok, keep, a, s_ids, fn, lane);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t) bt[s][t] = wide_operand(tk, t, s);
      wide_issue_tok(tk, a, m0, fn, lane);
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      char* slot = my_slots + i * kSlot;
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kInFlight) : "memory");
      u32x4 wf[4];
      if constexpr (MX) {
        const Frag8 f8 = wide_read_w8_mx(slot, table_scales(stable, a, rw, i, fc, lane), lane);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wide_copy_w8(slot, a, rw, i, fn, live, lane);
        const int wsc = int((f8.sdw >> (8 * (lane >> 4))) & 0xFFu);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[i][t] = mfma_mx16x16x128(f8.c0, f8.c1, wsc, bx_lo[t], bx_hi[t], bx_sc[t], acc[i][t]);
      } else if constexpr (W8) {
        const Frag8 f8 = wide_read_w8(slot, table_scales(stable, a, rw, i, fc, lane), lane);
        // the slot is read (into registers) before its next copy is issued
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wide_copy_w8(slot, a, rw, i, fn, live, lane);
        wide_operands_w8(wf, f8, lane);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          wf[s] = *reinterpret_cast<const u32x4*>(slot + fl + 16 * ((4 * (lane >> 4) + s) ^ (lane & 15)));
        // the slot is read (into registers) before its next copy is issued
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wide_copy_w(slot, a, rw, i, fn, live, lane);
      }
      if constexpr (!MX) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[i][t] = mfma16x16x32(wf[s], bt[s][t], acc[i][t]);
      }
      asm volatile("" ::: "memory");
    }
  }
  // the refill copies after the last chunk land before the slots are reused
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The one-token-block decode loop with one more weight slot.  Where every workgroup's rows end
// in a block of at most four rows (100 rows: six full blocks and four rows), that block keeps
// only its four rows (a 1 KB slot, one copy per chunk), and the hash ids are staged as 32-bit
// values; the LDS this frees holds a second slot for row block 0, which is then copied two
// chunks ahead: a wave keeps NRB x 4 KB of rows in flight instead of (NRB - 1) x 4 KB and four
// rows.  Wave layout: slots of blocks 0 .. NRB - 2 (4 KB each), the last block's 1 KB slot,
// block 0's second slot (chunks c with c odd).
__host__ __device__ constexpr int deep_wave_bytes(int nrb) { return (nrb - 1) * kWBlk + 1024 + kWBlk; }
__host__ __device__ constexpr int deep_ids_off(int nrb) { return 4 * deep_wave_bytes(nrb) + 4 * kTokBuf_; }
__host__ __device__ constexpr int deep_lds_bytes(int nrb, int n_cols) {
  return deep_ids_off(nrb) + kTB * n_cols * 4 > nrb * 16384 ? deep_ids_off(nrb) + kTB * n_cols * 4 : nrb * 16384;
}

// The last row block's copy: its rows 0..3 (past the workgroup's last row: the last row), lane
// l at 16 l: row l / 16, part (l % 16) ^ row, as the first copy of a full block.  Not live:
// rows 0..3 at feature 0 (cache resident).
__device__ __forceinline__ void deep_copy_last(char* slot, const StreamArgs& a, const Rows& rw, int nrb, int f_chunk,
                                               bool live, int lane) {
  const int rr = lane >> 4;
  const int rbase = live ? rw.r0 + 16 * (nrb - 1) : 0;
  const int rlast = live ? rw.r1 - 1 : 3;
  const int r = rbase + rr;
  const size_t row = size_t(r < rlast ? r : rlast);
  const size_t fbase = live ? size_t(f_chunk) : 0;
  __builtin_amdgcn_global_load_lds((const void*)(a.wkv + row * a.K + fbase + 8 * ((lane & 15) ^ rr)),
                                   (lds_ptr_t)slot, 16, 0, 2);
}

template <int NRB>
__device__ __forceinline__ void deep_loop(f32x4 (&acc)[NRB][4], const StreamArgs& a, const int32_t* s_ids,
                                          char* smem, const Rows& rw, int lane, int wv) {
  static_assert(NRB >= 2, "a full block and the last one");
  const int q0 = wv * (a.K >> 2);
  const int nch = (a.K >> 2) / 128;
  const int rot = int((5u * blockIdx.x) % uint32_t(nch));
  auto feat = [&](int c) { return q0 + 128 * ((c + rot) % nch); };
  char* const base = smem + wv * deep_wave_bytes(NRB);
  char* const last_slot = base + (NRB - 1) * kWBlk;
  char* const b0_second = last_slot + 1024;
  char* const my_tok = smem + 4 * deep_wave_bytes(NRB) + wv * kTokBuf;
  uint32_t keep[4];
  // Copy order: chunk 0's tokens, block 0 of chunks 0 and 1, blocks 1 .. NRB - 1 of chunk 0; then
  // per chunk c: chunk c + 1's tokens (T copies), block 0 of chunk c + 2 (4), blocks 1 .. NRB - 2
  // of chunk c + 1 (4 each), the last block of chunk c + 1 (1).  So when a chunk's tokens are
  // waited for, only the next chunk's block 0 and this chunk's blocks 1 .. NRB - 1 may follow
  // them: 4 (NRB - 1) + 1; that wait also covers this chunk's block 0 (copied before them).
  // Block i in 1 .. NRB - 2 is followed by the rest of its chunk's blocks, 4 (NRB - 2 - i) + 1,
  // then the next tokens, T, block 0 two chunks ahead, 4, and blocks 1 .. i - 1 of the next
  // chunk, 4 (i - 1): 4 (NRB - 2) + 1 + T in all; the last block by T + 4 (NRB - 1).
  constexpr int T = kTokLoads<true, false>;
  constexpr int kTokWait = 4 * (NRB - 1) + 1;
  constexpr int kMidWait = 4 * (NRB - 2) + 1 + T;
  constexpr int kLastWait = T + 4 * (NRB - 1);
  static_assert(kMidWait <= 63 && kLastWait <= 63, "vmcnt range");
  wide_copy_tok<true, int32_t>(my_tok, keep, a, s_ids, feat(0), lane);
  asm volatile("" ::: "memory");
  wide_copy_w(base, a, rw, 0, feat(0), true, lane);
  asm volatile("" ::: "memory");
  wide_copy_w(b0_second, a, rw, 0, feat(nch > 1 ? 1 : 0), nch > 1, lane);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 1; i < NRB - 1; ++i) {
    wide_copy_w(base + i * kWBlk, a, rw, i, feat(0), true, lane);
    asm volatile("" ::: "memory");
  }
  deep_copy_last(last_slot, a, rw, NRB, feat(0), true, lane);
  asm volatile("" ::: "memory");
  const int fl = (lane & 15) * 256;  // this lane's fragment row in a full slot
  const int lr = (lane & 15) < 3 ? (lane & 15) : 3;  // ... and in the last block's slot
  for (int c = 0; c < nch; ++c) {
    const bool live = c + 1 < nch, live2 = c + 2 < nch;
    const int fc = feat(c);
    const int fn = feat(live ? c + 1 : c);
    const int fnn = feat(live2 ? c + 2 : c);
    u32x4 bt[4][4];
    // the token copies of chunk c (and block 0 of chunk c) have landed
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kTokWait) : "memory");
    const int cc_cur = fc % a.head_dim + 32 * (lane >> 4);
    const uint32_t e8m0_shift = uint32_t((cc_cur / a.scale_block) & 3) * 8u;
    wide_tok_operands(bt, my_tok, keep, lane, a.scale_e8m0, e8m0_shift);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the buffer is read before its refill
    wide_copy_tok<true, int32_t>(my_tok, keep, a, s_ids, fn, lane);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      const bool last = i == NRB - 1;
      char* slot = i == 0 ? ((c & 1) ? b0_second : base) : (last ? last_slot : base + i * kWBlk);
      if (i > 0) {
        if (last) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLastWait) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kMidWait) : "memory");
      }
      u32x4 wf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        wf[s] = last ? *reinterpret_cast<const u32x4*>(slot + lr * 256 + 16 * ((4 * (lane >> 4) + s) ^ lr))
                     : *reinterpret_cast<const u32x4*>(slot + fl + 16 * ((4 * (lane >> 4) + s) ^ (lane & 15)));
      // the slot is read (into registers) before its next copy is issued
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (i == 0) wide_copy_w(slot, a, rw, 0, fnn, live2, lane);
      else if (last) deep_copy_last(slot, a, rw, NRB, fn, live, lane);
      else wide_copy_w(slot, a, rw, i, fn, live, lane);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = mfma16x16x32(wf[s], bt[s][t], acc[i][t]);
      asm volatile("" ::: "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------------------ per token block
// Sums the four K-partials in wave order; afterwards wave wv holds token sub-block wv.  With
// ONE_ROUND (X holds NRB x 16 KB: the wide loop's weight slots) all row blocks pass through LDS
// at once, else two at a time.
// A workgroup barrier that completes only the wave's LDS accesses (no wait for memory).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int NRB, bool ONE_ROUND>
__device__ __forceinline__ void reduce_k(f32x4 (&red)[NRB], f32x4 (&acc)[NRB][4], f32x4* X, int cnt, int lane,
                                         int wv) {
  if constexpr (ONE_ROUND) {
    // (LDS-only barriers: the wide loop's copies have all landed, and the epilogue inputs loaded
    // just before stay in flight under the exchange; __syncthreads would wait for them.  The
    // wide kernels instantiate their blocks per row-block count, so cnt == NRB here: every
    // fragment is exchanged without a branch, and the reads are issued together.)
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) X[((i * 4 + wv) * 4 + t) * 64 + lane] = acc[i][t];
    lds_barrier();
    f32x4 p[NRB][4];
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) p[i][q] = X[((i * 4 + q) * 4 + wv) * 64 + lane];
#pragma unroll
    for (int i = 0; i < NRB; ++i) red[i] = ((p[i][0] + p[i][1]) + p[i][2]) + p[i][3];
    lds_barrier();  // X overlaps the epilogue's shared words
    return;
  }
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
}

struct Shared {
  float red[4][kTB][3];
  int last[2];
  int last2[2][2];  // the two-token-block kernel: last-arriver marks per (token block, stream slot)
  int last4[4][2];  // ... and the four-token-block kernel's
};

// The gate of token t from the four quarter sums in sh.red[q][t] (|h|^2, |key|^2, h q k key),
// added in quarter order: sigmoid of the signed square root of the clamped scaled dot product.
__device__ __forceinline__ float gate_from_quarters(const StreamArgs& a, const Shared& sh, int t) {
  const float A = ((sh.red[0][t][0] + sh.red[1][t][0]) + sh.red[2][t][0]) + sh.red[3][t][0];
  const float Kq = ((sh.red[0][t][1] + sh.red[1][t][1]) + sh.red[2][t][1]) + sh.red[3][t][1];
  const float D = ((sh.red[0][t][2] + sh.red[1][t][2]) + sh.red[2][t][2]) + sh.red[3][t][2];
  const float fd = float(a.dim);
  const float rstd = __frsqrt_rn(A / fd + a.eps) * __frsqrt_rn(Kq / fd + a.eps);
  const float dot = D * rstd * a.inv_sqrt_dim;
  const float z = copysignf(sqrtf(fmaxf(fabsf(dot), a.clamp)), dot);
  return 1.0f / (1.0f + expf(-z));
}

// Parts of the fused epilogue, so that a kernel with two token blocks can interleave them with
// its own: store the key columns' partial sums; count the workgroup in (last-arriver marks); the
// last arrivers' gates; the value columns.
constexpr int kPhStore = 1, kPhCount = 2, kPhGates = 4, kPhValue = 8, kPhAll = 15;
constexpr int kPhNoMark = 16;  // value tiles stored, ready marks left to the caller

// Inputs of the key columns' partial sums, loaded before the K-partial reduction: per row block,
// the lane's 4 features of x (token 16 wv + lane % 16, its stream) and the fp32 products q * k of
// those features.
template <int NRB>
struct KeyPre {
  u32x2 x[NRB];
  f32x4 wq[NRB];
};

template <int NRB>
__device__ __forceinline__ void prefetch_key(KeyPre<NRB>& kp, const StreamArgs& a, const Rows& rw, int64_t m0,
                                             int tid) {
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t m = m0 + 16 * wv + (lane & 15);
  const int64_t mm = m < a.M ? m : a.M - 1;
  // the workgroup's rows span at most two streams (checked on the host): seg_lo and seg_lo + 1
  const int seg_lo = rw.r0 / a.dim;
  const int nb1 = (seg_lo + 1) * a.dim;
#pragma unroll
  for (int i = 0; i < NRB; ++i) {
    int n = rw.r0 + 16 * i + 4 * (lane >> 4);
    n = n < rw.r1 ? n : rw.r1 - 4;
    const int s0 = n < nb1 ? seg_lo : seg_lo + 1;
    const int s = s0 < 4 ? s0 : 3;  // value columns: unused, any in-range address
    const int d = n - s0 * a.dim;
    kp.x[i] = *reinterpret_cast<const u32x2*>(a.x + (mm * 4 + s) * a.dim + d);
    const f32x4 q4 = *reinterpret_cast<const f32x4*>(a.q_weight + s * a.dim + d);
    const f32x4 k4 = *reinterpret_cast<const f32x4*>(a.k_weight + s * a.dim + d);
    kp.wq[i] = f32x4{q4.x * k4.x, q4.y * k4.y, q4.z * k4.z, q4.w * k4.w};
  }
}

// The same for another token block whose products q * k are those of `same` (loaded before).
template <int NRB>
__device__ __forceinline__ void prefetch_key_x(KeyPre<NRB>& kp, const StreamArgs& a, const Rows& rw, int64_t m0,
                                               int tid, const KeyPre<NRB>& same) {
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t m = m0 + 16 * wv + (lane & 15);
  const int64_t mm = m < a.M ? m : a.M - 1;
  const int seg_lo = rw.r0 / a.dim;
  const int nb1 = (seg_lo + 1) * a.dim;
#pragma unroll
  for (int i = 0; i < NRB; ++i) {
    int n = rw.r0 + 16 * i + 4 * (lane >> 4);
    n = n < rw.r1 ? n : rw.r1 - 4;
    const int s0 = n < nb1 ? seg_lo : seg_lo + 1;
    const int s = s0 < 4 ? s0 : 3;
    kp.x[i] = *reinterpret_cast<const u32x2*>(a.x + (mm * 4 + s) * a.dim + (n - s0 * a.dim));
    kp.wq[i] = same.wq[i];
  }
}

// Cross-workgroup control words: one counter per (token block, stream) on its own 256-byte
// line (contended atomics on one line serialise).
// The workspace holds one block per token block at a fixed stride (so, for one layout, every
// control word sits at the same offset whatever the token count):
//   [4 counters, 256 B apart][gate slots: grid x 4 x 64 words][partials: grid x 2 x 64 x 16 B]
__device__ __forceinline__ uint32_t* tb_block(const StreamArgs& a, int64_t tb) {
  return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(a.ws_hdr) + 256 + size_t(tb) * a.tb_stride);
}
__device__ __forceinline__ uint32_t* counter_of(const StreamArgs& a, int64_t tb, int s) {
  return tb_block(a, tb) + s * 64;
}
// Partial sums of workgroup w for its stream slot sl: 64 records of 16 bytes (|h|^2, |key|^2,
// h q k key, 0), as a byte offset from the workspace start (they are accessed through a buffer
// resource on it).
__device__ __forceinline__ uint32_t partial_off(const StreamArgs& a, int64_t tb, int w, int sl) {
  return uint32_t(256 + size_t(tb) * a.tb_stride + (256 + size_t(a.G) * 4 * kTB) * 4 +
                  (size_t(w) * 2 + sl) * (kTB * 16));
}
// Gate slot of value workgroup w for stream s: 64 words, written once by the stream's last
// arriver (value bits with the sign bit set), read and cleared by w alone.
__device__ __forceinline__ uint32_t* gate_slot(const StreamArgs& a, int64_t tb, int w, int s) {
  return tb_block(a, tb) + 256 + (size_t(w) * 4 + s) * kTB;
}

// Apply workgroups (the fused forward of one token block, and of two in the two-token-block
// kernel).  Value workgroup j (the j-th from the first one that owns a value row) does not wait
// for the gates: for each token block it leaves its bf16 values in a tile behind the token
// blocks' part of the workspace, one kVRow-byte row per token (its value features, shifted by 0
// or 4 features so that 16-byte pieces line up with those of x and out), and marks the tile
// ready; apply workgroup 2 j + h of the block, among the last ids of the grid, applies the gates
// to tokens 32 h .. 32 h + 31 of it.  The apply workgroups run on the CUs that the key
// workgroups leave, and the value workgroups' output work (64 tokens x 4 streams of their
// features, issue-bound on one wave per SIMD) is spread over twice as many workgroups.  Slot k of
// an apply workgroup (32 words, in its token block's gate-slot region): k = 0..3 the gates of
// stream k for its 32 tokens, k = 4 word 0 the tile's ready mark; each written once by its
// producer, read and cleared by that workgroup alone, which also clears its half of the tile.
constexpr int kVRow = 240;            // bytes per token row of a value tile (up to 120 features)
constexpr int kVTile = kTB * kVRow;   // one value workgroup's tile
__device__ __forceinline__ uint32_t* apply_slot(const StreamArgs& a, int64_t tb, int ap, int k) {
  return tb_block(a, tb) + 256 + (size_t(ap) * 5 + k) * 32;
}
// value workgroup j's tile of token block tb, behind the n_atb token blocks' control words
__device__ __forceinline__ uint32_t vtile_off(const StreamArgs& a, int64_t tb, int j) {
  const int V = a.n_apply / (2 * a.n_atb);
  return uint32_t(256 + size_t(a.n_atb) * a.tb_stride + (size_t(tb) * V + j) * kVTile);
}
__device__ __forceinline__ uint32_t ws_off(const StreamArgs& a, const uint32_t* p) {
  return uint32_t(reinterpret_cast<const char*>(p) - reinterpret_cast<const char*>(a.ws_hdr));
}

// Value workgroups of the wide kernel write their output rows through LDS (stage_bytes at the
// start of the LDS, which then holds no live data except the gates in Shared, read before it is
// overwritten).  In the MFMA layout a store instruction writes 8 bytes for each of 16 tokens (16
// separate 32-byte runs); from LDS, each instruction writes 16 bytes per lane along 4 rows (4
// contiguous runs of up to 256 bytes), and half as many instructions are issued.  Row (s, token)
// of a wave's 64 rows holds the workgroup's value features of that row, shifted by `shift`
// features so that the 16-byte pieces line up with 16-byte global addresses.
__host__ __device__ constexpr int stage_row_bytes(int nrb) { return 32 * nrb + 16; }
__host__ __device__ constexpr int stage_bytes(int nrb) { return 4 * 64 * stage_row_bytes(nrb) + 256; }

template <int NRB, bool FUSED, bool STAGE = false, bool APPLY = false, int PH = kPhAll>
__device__ __forceinline__ void epilogue(const StreamArgs& a, f32x4 (&red)[NRB], const KeyPre<NRB>& kp, Shared& sh,
                                         int64_t tb, int w,
                                         const Rows& rw, int tid, char* stage = nullptr) {
  const int lane = tid & 63, wv = tid >> 6;
  int* const lf = sh.last;
  const int G = a.G;
  const int Q = a.N >> 2;
  const __amdgpu_buffer_rsrc_t wsr = coherent_rsrc(a.ws_hdr);
  const int cnt = rw.nblk;
  const int seg_lo = rw.r0 / a.dim;
  const int seg_hi = (rw.r1 - 1) / a.dim;
  // (at most two streams per workgroup: a row is in seg_lo below nb1; value rows from nv on.
  // Comparisons, not divisions: this code runs once per call, cold in the instruction cache)
  const int nb1 = (seg_lo + 1) * a.dim;
  const int nv = 4 * a.dim;
  const int64_t m0 = tb * kTB;
  const int tok = 16 * wv + (lane & 15);
  const int64_t m = m0 + tok;
  const bool mvalid = m < a.M;

  if constexpr (!FUSED) {
    if (mvalid) {
#pragma unroll
      for (int i = 0; i < NRB; ++i) {
        const int n = rw.r0 + 16 * i + 4 * (lane >> 4);  // four columns, all in [r0, r1) or none
        if (i < cnt && n < rw.r1)
          *reinterpret_cast<u32x2*>(a.kv + m * a.N + n) =
              u32x2{pack_bf16x2(red[i].x, red[i].y), pack_bf16x2(red[i].z, red[i].w)};
      }
    }
    return;
  } else {
    // ---- key columns: per-token partial sums for up to two streams
    float pa[2] = {0.f, 0.f}, pk[2] = {0.f, 0.f}, pd[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      const int n = rw.r0 + 16 * i + 4 * (lane >> 4);
      // (dim is a multiple of 4: the lane's four columns share a stream)
      if (i < cnt && n < rw.r1) {
        if (n < nv) {
          const float key[4] = {bf16_round(red[i].x), bf16_round(red[i].y), bf16_round(red[i].z),
                                bf16_round(red[i].w)};
          const u32x2 xw = mvalid ? kp.x[i] : u32x2{0u, 0u};
          const float h[4] = {bf16_lo(xw.x), bf16_hi(xw.x), bf16_lo(xw.y), bf16_hi(xw.y)};
          const float wq[4] = {kp.wq[i].x, kp.wq[i].y, kp.wq[i].z, kp.wq[i].w};
          float sa = 0.f, sk = 0.f, sd = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sa += h[r] * h[r];
            sk += key[r] * key[r];
            sd += (h[r] * wq[r]) * key[r];
          }
          if (n < nb1) {
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
      if constexpr ((PH & kPhStore) != 0) {
        if (lane < 16) {
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) {
            if (seg_lo + sl <= seg_hi && seg_lo + sl < 4) {
              store_coherent4(wsr, partial_off(a, tb, w, sl) + tok * 16, f32x4{pa[sl], pk[sl], pd[sl], 0.f});
            }
          }
        }
      }
      if constexpr ((PH & kPhCount) != 0) {
        drain_memory_ops();
        __syncthreads();
        if (tid == 0) {
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) {
            const int s = seg_lo + sl;
            lf[sl] = 0;
            if (s <= seg_hi && s < 4) {
              const int wf = owner_of_row(s * a.dim, Q, G), wl = owner_of_row((s + 1) * a.dim - 1, Q, G);
              const uint32_t old = atomic_add_relaxed(counter_of(a, tb, s), 1u);
              lf[sl] = (old == uint32_t(wl - wf)) ? 1 : 0;
            }
          }
        }
        __syncthreads();
      }
#pragma unroll 1
      for (int sl = 0; sl < 2; ++sl) {
        if ((PH & kPhGates) != 0 && lf[sl]) {
          __syncthreads();  // sh.red may still be read for the other stream
          // every contributor has posted: sum the partials in workgroup order
          const int s = seg_lo + sl;
          const int wf = owner_of_row(s * a.dim, Q, G), wl = owner_of_row((s + 1) * a.dim - 1, Q, G);
          const int nW = wl - wf + 1;
          const int t = tid & 63, q = tid >> 6;
          const int wb0 = wf + (nW * q) / 4, wb1 = wf + (nW * (q + 1)) / 4;
          // a contributor's slot for stream s: the second for the first contributor when its rows
          // begin in stream s - 1, else the first
          const int sl_f = row_begin(wf, Q, G) < s * a.dim ? 1 : 0;
          auto poff = [&](int w2) { return partial_off(a, tb, w2, w2 == wf ? sl_f : 0) + t * 16; };
          // all loads of a group of 16 contributors are issued before any is used (one
          // memory round trip per group, not one per contributor); sums stay in order
          float ra = 0.f, rk = 0.f, rd = 0.f;
          for (int base = wb0; base < wb1; base += 16) {
            f32x4 v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
              v[k] = load_coherent4(wsr, poff(base + k < wb1 ? base + k : wb0));
            }
#pragma unroll
            for (int k = 0; k < 16; ++k) {
              if (base + k < wb1) {
                ra += v[k].x;
                rk += v[k].y;
                rd += v[k].z;
              }
            }
          }
          sh.red[q][t][0] = ra;
          sh.red[q][t][1] = rk;
          sh.red[q][t][2] = rd;
          __syncthreads();
          // (closed tokens keep x: the value workgroups apply the mask)
          if (q == 0) sh.red[0][t][0] = m0 + t < a.M ? gate_from_quarters(a, sh, t) : 0.0f;
          __syncthreads();
          // this call is done with the counter; hand the 64 gates to every value workgroup in
          // its own slot, sign bit set as the ready mark (gates are >= 0)
          if (tid == 0) store_relaxed(counter_of(a, tb, s), 0u);
          const int v0 = owner_of_row(4 * a.dim, Q, G);
          // four words per 16-byte device-coherent store
          if constexpr (APPLY) {
            // apply workgroup ap of the block takes tokens 32 (ap & 1) .. + 31
            for (int i = tid; i < (a.n_apply / a.n_atb) * 8; i += 256) {
              const int ap = i >> 3, t4 = 32 * (ap & 1) + 4 * (i & 7);
              store_coherent4(wsr, ws_off(a, apply_slot(a, tb, ap, s) + 4 * (i & 7)),
                              __builtin_bit_cast(f32x4, u32x4{__float_as_uint(sh.red[0][t4][0]) | 0x80000000u,
                                                              __float_as_uint(sh.red[0][t4 + 1][0]) | 0x80000000u,
                                                              __float_as_uint(sh.red[0][t4 + 2][0]) | 0x80000000u,
                                                              __float_as_uint(sh.red[0][t4 + 3][0]) | 0x80000000u}));
            }
          } else
          for (int i = tid; i < (G - v0) * (kTB / 4); i += 256) {
            const int v = v0 + i / (kTB / 4), t4 = 4 * (i % (kTB / 4));
            const uint32_t off = uint32_t(reinterpret_cast<char*>(gate_slot(a, tb, v, s) + t4) -
                                          reinterpret_cast<char*>(a.ws_hdr));
            store_coherent4(wsr, off,
                            __builtin_bit_cast(f32x4, u32x4{__float_as_uint(sh.red[0][t4][0]) | 0x80000000u,
                                                            __float_as_uint(sh.red[0][t4 + 1][0]) | 0x80000000u,
                                                            __float_as_uint(sh.red[0][t4 + 2][0]) | 0x80000000u,
                                                            __float_as_uint(sh.red[0][t4 + 3][0]) | 0x80000000u}));
          }
          // the partials are consumed: leave them zero, so that the whole workspace is zero
          // again after the call (any schedule may use it next)
          for (int w2 = wb0; w2 < wb1; ++w2) store_coherent4(wsr, poff(w2), f32x4{0.f, 0.f, 0.f, 0.f});
        }
      }
    }

    if constexpr ((PH & kPhValue) == 0) return;
    // ---- value columns, apply workgroups present: the bf16 values into this workgroup's tile
    if constexpr (APPLY) {
      if (seg_hi == 4) {
        const int j = w - owner_of_row(4 * a.dim, Q, G);
        const int cv_lo = rw.r0 > nv ? rw.r0 : nv;
        const int shift = (cv_lo - nv) & 7;
        const uint32_t row = vtile_off(a, tb, j) + uint32_t(tok) * kVRow;
#pragma unroll
        for (int i = 0; i < NRB; ++i) {
          const int n = rw.r0 + 16 * i + 4 * (lane >> 4);
          if (i < cnt && n < rw.r1 && n >= nv)
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2{pack_bf16x2(red[i].x, red[i].y), pack_bf16x2(red[i].z, red[i].w)}, wsr,
                row + 2 * uint32_t(n - cv_lo + shift), 0, kCpolSc1);
        }
        if constexpr ((PH & kPhNoMark) == 0) {
          drain_memory_ops();
          __syncthreads();
          if (tid < 2) store_relaxed(apply_slot(a, tb, 2 * j + tid, 4), 0x80000000u);
        }
      }
      return;
    }
    // ---- value columns: wait for the four gates, then out = h + g * value on every stream
    if (seg_hi == 4) {
      // the streams of this workgroup's features are read before waiting
      u32x2 xs[NRB][4];
#pragma unroll
      for (int i = 0; i < NRB; ++i) {
        const int n = rw.r0 + 16 * i + 4 * (lane >> 4);
        if (i < cnt && n < rw.r1 && n >= nv && mvalid) {
          const int d = n - nv;
#pragma unroll
          for (int s = 0; s < 4; ++s) xs[i][s] = *reinterpret_cast<const u32x2*>(a.x + size_t(m * 4 + s) * a.dim + d);
        }
      }
      const bool open = mvalid && (a.token_mask == nullptr || a.token_mask[m] != 0);
      __syncthreads();  // sh.red may still be read by a last-arriver hand-off above
      {
        // thread (s, t) waits for gate t of stream s in this workgroup's slot, then clears it.
        // (A wave's poll is one 256-byte read, and each poll waits for its read to return, so
        // the 4 x 51 polling waves add ~50 GB/s at most to the memory system.)
        const int s = tid >> 6, t = tid & 63;
        uint32_t* slot = gate_slot(a, tb, w, s) + t;
        uint32_t bits = 0u;
        uint32_t it = 0;
        while ((bits = load_relaxed(slot)) == 0u) {
          __builtin_amdgcn_s_sleep(2);
          if (++it > a.spin_budget) {
            atomic_add_relaxed(&a.ws_hdr[0], 1u);
            break;
          }
        }
        store_relaxed(slot, 0u);
        sh.red[s][t][0] = __uint_as_float(bits & 0x7FFFFFFFu);
      }
      __syncthreads();
      float g[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) g[s] = sh.red[s][tok][0];
      if constexpr (STAGE) {
        const int cv_lo = rw.r0 > nv ? rw.r0 : nv;  // first value row of this workgroup
        const int nc = rw.r1 - cv_lo;               // its value features (a multiple of 4)
        const int shift = (cv_lo - nv) & 7;         // 0 or 4
        constexpr int rs = stage_row_bytes(NRB);
        char* const stg = stage + wv * (64 * rs);
        // bit t: token 16 wv + t is written (lanes 0..15 hold tokens 0..15 of the wave)
        const uint64_t keep = __ballot(lane < 16 && mvalid && (open || a.out != a.x));
        lds_barrier();  // every wave has read its gates: the staging covers Shared
        if (mvalid) {
#pragma unroll
          for (int i = 0; i < NRB; ++i) {
            const int n = rw.r0 + 16 * i + 4 * (lane >> 4);
            if (i < cnt && n < rw.r1 && n >= nv) {
              const int c = n - cv_lo + shift;
              const float v[4] = {bf16_round(red[i].x), bf16_round(red[i].y), bf16_round(red[i].z),
                                  bf16_round(red[i].w)};
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                const u32x2 xw = xs[i][s];
                u32x2 o = xw;
                if (open) {
                  o.x = pack_bf16x2(bf16_lo(xw.x) + g[s] * v[0], bf16_hi(xw.x) + g[s] * v[1]);
                  o.y = pack_bf16x2(bf16_lo(xw.y) + g[s] * v[2], bf16_hi(xw.y) + g[s] * v[3]);
                }
                // rows stream-major: the 16 tokens of a write fall on distinct bank pairs
                *reinterpret_cast<u32x2*>(stg + (s * 16 + (lane & 15)) * rs + 2 * c) = o;
              }
            }
          }
        }
        // (a wave reads only its own rows: its LDS accesses complete in order.)  Lane l covers
        // features 8 (l % 16) .. of row 4 it + l / 16: both halves, the lower or the upper four.
        const int rr = lane >> 4, pc = 8 * (lane & 15);
        const bool lo_ok = pc >= shift && pc + 4 <= shift + nc;
        const bool hi_ok = pc + 4 >= shift && pc + 8 <= shift + nc;
        const size_t col0 = size_t(cv_lo - nv - shift + pc);
        u32x4 piece[16];
#pragma unroll
        for (int it = 0; it < 16; ++it) piece[it] = *reinterpret_cast<const u32x4*>(stg + (4 * it + rr) * rs + 2 * pc);
#pragma unroll
        for (int it = 0; it < 16; ++it) {
          const int s = it >> 2, tt = 4 * (it & 3) + rr;  // row 4 it + rr = 16 s + tt
          if ((keep >> tt) & 1u) {
            uint16_t* dst = a.out + size_t((m0 + 16 * wv + tt) * 4 + s) * a.dim + col0;
            if (lo_ok && hi_ok) *reinterpret_cast<u32x4*>(dst) = piece[it];
            else if (lo_ok) *reinterpret_cast<u32x2*>(dst) = u32x2{piece[it].x, piece[it].y};
            else if (hi_ok) *reinterpret_cast<u32x2*>(dst + 4) = u32x2{piece[it].z, piece[it].w};
          }
        }
      } else if (mvalid) {
#pragma unroll
        for (int i = 0; i < NRB; ++i) {
          const int n = rw.r0 + 16 * i + 4 * (lane >> 4);
          if (i < cnt && n < rw.r1 && n >= nv) {
            const int d = n - nv;
            const float v[4] = {bf16_round(red[i].x), bf16_round(red[i].y), bf16_round(red[i].z),
                                bf16_round(red[i].w)};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const size_t off = size_t(m * 4 + s) * a.dim + d;
              const u32x2 xw = xs[i][s];
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
  }
}

// One 64-token block: stage the hash ids, run the K loop, reduce, finish.
template <int NRB, bool WIDE, int U, bool FUSED, bool W8 = false, bool MX = false, bool APPLY = false,
          bool DEEP = false>
__device__ __forceinline__ void token_block(const StreamArgs& a, char* smem, Shared& sh, int64_t tb, int w,
                                            const Rows& rw) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t m0 = tb * kTB;
  int64_t* const s_ids = reinterpret_cast<int64_t*>(smem + (WIDE ? wide_lds_bytes(NRB, FUSED, W8) : kRedBytes));
  // the deep decode loop stages the ids as 32-bit values behind its own layout
  int32_t* const s_ids32 = reinterpret_cast<int32_t*>(smem + deep_ids_off(NRB));
  // MXFP8 weights: the table of the workgroup's weight scales behind the staged ids, loaded with
  // the first token block (with the hash ids' loads in flight, in the fused kernel)
  char* const stable = reinterpret_cast<char*>(s_ids) + (FUSED ? kTB * a.n_cols * 8 : 0);
  // MX: the waves' token-scale tables behind the weight-scale table
  char* const ttable = stable + (((rw.r1 - rw.r0) * (a.K / 32) + 15) & ~15) + (MX ? wv * tok_table_bytes(a) : 0);
  if constexpr (W8) {
    if (tb == 0) {
      load_scale_table(stable, a, rw, tid);
      if constexpr (!FUSED) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
    }
  }
  KeyPre<NRB> kp;
  if constexpr (FUSED) {
    // hash ids of the token block, checked once: -1 marks a row that reads as zeros.  Eight
    // loads per thread are in flight at a time.
    const int n_ids = kTB * a.n_cols;
    const int64_t n_valid = (a.M - m0 < kTB ? a.M - m0 : kTB) * a.n_cols;
    for (int base = 0; base < n_ids; base += 8 * 256) {
      int64_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = base + q * 256 + tid;
        v[q] = i < n_valid ? a.hash_ids[m0 * a.n_cols + i] : -1;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = base + q * 256 + tid;
        int64_t r = v[q];
        if (i < n_valid && (r < 0 || r >= a.n_rows)) {
          if (w == 0 && a.err_count != nullptr) atomicAdd(a.err_count, 1);
          r = -1;
        }
        if (i < n_ids) {
          if constexpr (DEEP) s_ids32[i] = int32_t(r);
          else s_ids[i] = r;
        }
      }
    }
    // (the scale table's copies of every wave have landed before the barrier)
    if constexpr (W8) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if constexpr (MX) load_tok_scales(ttable, a, s_ids, wv * (a.K >> 2), lane);
  }
  f32x4 acc[NRB][4];
#pragma unroll
  for (int i = 0; i < NRB; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (DEEP) deep_loop<NRB>(acc, a, s_ids32, smem, rw, lane, wv);
  else if constexpr (WIDE) wide_loop<NRB, FUSED, W8, MX>(acc, a, s_ids, smem, stable, ttable, m0, rw, lane, wv);
  else narrow_loop<NRB, U, FUSED>(acc, a, s_ids, m0, rw, lane, wv);
  // the key columns' epilogue inputs are loaded now, so that their latency hides under the
  // K-partial reduction (loaded before the K loop they slow it down: registers)
  if constexpr (FUSED) prefetch_key<NRB>(kp, a, rw, m0, tid);
  f32x4 red[NRB];
  static_assert(!WIDE || DEEP || stage_bytes(NRB) <= wide_lds_bytes(NRB, FUSED, W8), "output staging exceeds the LDS");
  static_assert(!DEEP || (APPLY && FUSED && !W8), "the deep loop: fused, bf16 weights, apply workgroups");
  reduce_k<NRB, WIDE>(red, acc, reinterpret_cast<f32x4*>(smem), rw.nblk, lane, wv);
  epilogue<NRB, FUSED, WIDE, APPLY>(a, red, kp, sh, tb, w, rw, tid, smem);
  __syncthreads();
}

// Narrow kernel: NRB is the maximum row-block count per workgroup.
template <int NRB, int U, bool FUSED>
__global__ __launch_bounds__(256, 1) void k_stream_narrow(StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // the epilogue's shared words live behind the reduction buffer, in LDS the K loop no longer uses
  Shared& sh = *reinterpret_cast<Shared*>(smem + kRedBytes);
  const int G = a.G, w = blockIdx.x;
  const Rows rw = rows_of(w, a.N, G);
  const int64_t n_tb = (a.M + kTB - 1) / kTB;
  for (int64_t tb = 0; tb < n_tb; ++tb) token_block<NRB, false, U, FUSED>(a, smem, sh, tb, w, rw);
}

// Apply workgroup ap (value tile j = ap / 2, tokens 32 (ap & 1) .. + 31): out = h + g * value
// on all four streams of the tile's features.  Thread pairs (token t, 16-byte piece p) of the
// rows, t = idx / 16 and p = idx % 16 for idx = tid, tid + 256; x is loaded before waiting.
__device__ __forceinline__ void apply_wg(const StreamArgs& a, char* smem, int apg) {
  const int tid = threadIdx.x, G = a.G, Q = a.N >> 2;
  const int napb = a.n_apply / a.n_atb;  // apply workgroups per token block
  const int b = apg / napb, ap = apg - b * napb;
  const int j = ap >> 1, th = ap & 1;
  const Rows rw = rows_of(owner_of_row(4 * a.dim, Q, G) + j, a.N, G);
  const int nv = 4 * a.dim;
  const int cv_lo = rw.r0 > nv ? rw.r0 : nv, nc = rw.r1 - cv_lo, shift = (cv_lo - nv) & 7;
  const __amdgpu_buffer_rsrc_t wsr = coherent_rsrc(a.ws_hdr);
  float* const gl = reinterpret_cast<float*>(smem);  // gates [stream][token]
  u32x4 xv[2][4];
  bool lo_ok[2], hi_ok[2], open[2];
  size_t col[2];
  int64_t m[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + 256 * k, t = idx >> 4, pc = 8 * (idx & 15);
    m[k] = int64_t(b) * kTB + 32 * th + t;
    const bool mv = m[k] < a.M;
    lo_ok[k] = mv && pc >= shift && pc + 4 <= shift + nc;
    hi_ok[k] = mv && pc + 4 >= shift && pc + 8 <= shift + nc;
    col[k] = size_t(cv_lo - nv - shift + pc);
    open[k] = mv && (a.token_mask == nullptr || a.token_mask[m[k]] != 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint16_t* src = a.x + size_t(m[k] * 4 + s) * a.dim + col[k];
      xv[k][s] = u32x4{0u, 0u, 0u, 0u};
      if (lo_ok[k] && hi_ok[k]) xv[k][s] = *reinterpret_cast<const u32x4*>(src);
      else if (lo_ok[k]) { const u32x2 h = *reinterpret_cast<const u32x2*>(src); xv[k][s].x = h.x; xv[k][s].y = h.y; }
      else if (hi_ok[k]) { const u32x2 h = *reinterpret_cast<const u32x2*>(src + 4); xv[k][s].z = h.x; xv[k][s].w = h.y; }
    }
  }
  // the tile is ready, then the gates (each waited for by one thread, bounded)
  if (tid == 0) {
    uint32_t* flag = apply_slot(a, b, ap, 4);
    uint32_t it = 0;
    while (load_relaxed(flag) == 0u) {
      __builtin_amdgcn_s_sleep(2);
      if (++it > a.spin_budget) {
        atomic_add_relaxed(&a.ws_hdr[0], 1u);
        break;
      }
    }
    store_relaxed(flag, 0u);
  }
  __syncthreads();
  f32x4 vv[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    // (pieces that hold a feature end inside the row: 8 p + 4 <= shift + nc <= 116)
    vv[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lo_ok[k] || hi_ok[k])
      vv[k] = load_coherent4(wsr, vtile_off(a, b, j) + uint32_t(m[k] - int64_t(b) * kTB) * kVRow +
                                       16 * uint32_t((tid + 256 * k) & 15));
  }
  if (tid < 128) {
    const int s = tid >> 5, t = tid & 31;
    uint32_t* slot = apply_slot(a, b, ap, s) + t;
    uint32_t bits = 0u, it = 0;
    while ((bits = load_relaxed(slot)) == 0u) {
      __builtin_amdgcn_s_sleep(2);
      if (++it > a.spin_budget) {
        atomic_add_relaxed(&a.ws_hdr[0], 1u);
        break;
      }
    }
    store_relaxed(slot, 0u);
    gl[s * 32 + t] = __uint_as_float(bits & 0x7FFFFFFFu);
  }
  __syncthreads();
  // the eight gates first (one LDS round trip), then branch-free stores: a half piece that is
  // not written goes to an offset past the end of out, which the buffer store drops
  float g[2][4];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int s = 0; s < 4; ++s) g[k][s] = gl[s * 32 + ((tid + 256 * k) >> 4)];
  const size_t out_bytes = size_t(a.M) * 4 * size_t(a.dim) * 2;
  const __amdgpu_buffer_rsrc_t outr = __builtin_amdgcn_make_buffer_rsrc(
      a.out, (short)0, int(out_bytes < 0x7FFFFFFFu ? out_bytes : 0x7FFFFFFFu), 0x00020000);
  const bool wr = a.out != a.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const u32x4 v4 = __builtin_bit_cast(u32x4, vv[k]);
    const float v[8] = {bf16_lo(v4.x), bf16_hi(v4.x), bf16_lo(v4.y), bf16_hi(v4.y),
                        bf16_lo(v4.z), bf16_hi(v4.z), bf16_lo(v4.w), bf16_hi(v4.w)};
    const bool st = open[k] || wr;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float gs = open[k] ? g[k][s] : 0.0f;
      const u32x4 xw = xv[k][s];
      u32x4 o;
      o.x = pack_bf16x2(bf16_lo(xw.x) + gs * v[0], bf16_hi(xw.x) + gs * v[1]);
      o.y = pack_bf16x2(bf16_lo(xw.y) + gs * v[2], bf16_hi(xw.y) + gs * v[3]);
      o.z = pack_bf16x2(bf16_lo(xw.z) + gs * v[4], bf16_hi(xw.z) + gs * v[5]);
      o.w = pack_bf16x2(bf16_lo(xw.w) + gs * v[6], bf16_hi(xw.w) + gs * v[7]);
      if (!open[k]) o = xw;  // closed tokens pass through unchanged (a select, not a branch)
      const uint32_t off = uint32_t((size_t(m[k] * 4 + s) * a.dim + col[k]) * 2);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{o.x, o.y}, outr, st && lo_ok[k] ? off : 0xFFFFFFF0u, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{o.z, o.w}, outr, st && hi_ok[k] ? off + 8 : 0xFFFFFFF0u, 0, 0);
    }
  }
  // every thread's tile loads have returned (their values are used above): clear this half
  __syncthreads();
  for (int i = tid; i < 32 * kVRow / 16; i += 256)
    store_coherent4(wsr, vtile_off(a, b, j) + uint32_t(32 * th) * kVRow + 16 * uint32_t(i), f32x4{0.f, 0.f, 0.f, 0.f});
}

// Wide kernel: every workgroup has NLO or NHI = NLO + 1 row blocks, each compiled exactly (only
// one path when every workgroup has the same count, so registers are sized for it alone).
// ONE_TB: the call has a single token block.  Without a loop over token blocks the compiler
// has nothing to hoist above the hash-id loads; with one it computes every loop-invariant
// address of the K loop and the epilogue first, about 3 us before the first memory access.
template <int NLO, int NHI, bool FUSED, bool ONE_TB, bool W8, bool MX = false, bool DEEP = false>
__global__ __launch_bounds__(256, 1) void k_stream_wide(StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // the epilogue's shared words live behind the reduction buffer, in LDS the K loop no longer uses
  Shared& sh = *reinterpret_cast<Shared*>(smem + kRedBytes);
  const int G = a.G, w = blockIdx.x;
  if constexpr (ONE_TB && FUSED) {
    if (w >= G) {
      apply_wg(a, smem, w - G);
      return;
    }
  }
  const Rows rw = rows_of(w, a.N, G);
  if constexpr (ONE_TB) {
    if constexpr (DEEP) {
      static_assert(NLO == NHI, "the deep loop: one row-block count");
      token_block<NLO, true, 1, true, false, false, true, true>(a, smem, sh, 0, w, rw);
    } else if constexpr (NLO == NHI) {
      token_block<NLO, true, 1, FUSED, W8, MX, FUSED>(a, smem, sh, 0, w, rw);
    } else {
      if (rw.nblk == NLO) token_block<NLO, true, 1, FUSED, W8, MX, FUSED>(a, smem, sh, 0, w, rw);
      else token_block<NHI, true, 1, FUSED, W8, MX, FUSED>(a, smem, sh, 0, w, rw);
    }
    return;
  }
  const int64_t n_tb = (a.M + kTB - 1) / kTB;
  for (int64_t tb = 0; tb < n_tb; ++tb) {
    if constexpr (NLO == NHI) {
      token_block<NLO, true, 1, FUSED, W8, MX>(a, smem, sh, tb, w, rw);
    } else {
      if (rw.nblk == NLO) token_block<NLO, true, 1, FUSED, W8, MX>(a, smem, sh, tb, w, rw);
      else token_block<NHI, true, 1, FUSED, W8, MX>(a, smem, sh, tb, w, rw);
    }
  }
}

// ------------------------------------------------------------------------------ two token blocks
// The fused forward of 65..128 tokens in one pass over the weights, the one-block kernel's
// layout kept (one workgroup per CU over its row blocks, four waves each on a K quarter, every
// wave streaming its own weight rows, no barrier in the K loop) with two 64-token blocks per
// wave: chunks of 64 features, so that a wave's two stages of weight slots (2 x NRB x 2 KB) and
// its tokens' codes (128 tokens x 64 bytes, and their scales) fit the LDS together.  Per chunk a
// wave reads and dequantises its token operands, issues the next chunk's token copies, then
// refills each row block's slot with the rows two chunks ahead right after reading it, and
// multiplies NRB x 2 x 8 MFMAs.  Afterwards both token blocks go through the K-partial
// reduction and the key hand-off together; the value workgroups leave bf16 tiles for the apply
// workgroups, as in the one-block kernel.
constexpr int kC2 = 64;                 // features per chunk
constexpr int kW2Slot = 16 * kC2 * 2;   // LDS slot of one row block (2 KB)
constexpr int kTok2 = 2 * kTB * kC2 + 4 * 256;  // per wave: 128 tokens' codes, 2 x 128 scales
// LDS: two weight stages per wave (NRB slots each), the waves' token buffers, then the staged
// 32-bit hash ids of both token blocks; after the loop the K-partial reduction's NRB x 16 KB.
__host__ __device__ constexpr int tb2_lds(int nrb, int n_cols) {
  return (8 * nrb * kW2Slot + 4 * kTok2 + 2 * kTB * n_cols * 4) > nrb * 16384
             ? 8 * nrb * kW2Slot + 4 * kTok2 + 2 * kTB * n_cols * 4
             : nrb * 16384;
}

// Weight copy h of row block i: rows 8 h .. 8 h + 7, lane l at 16 l: row 8 h + l / 8, position
// l % 8, holding the 16-byte part (l % 8) ^ (row & 7) of the row's 128 chunk bytes.  The copies
// go through a buffer resource on wkv: a lane's byte offset of its row and part in row block 0,
// and in the workgroup's last row (rows past it repeat it), are computed once; the chunk's byte
// offset is a scalar.  Not live (after the last chunk): rows 0..15 at feature 0, a
// cache-resident 2 KB.
struct Tb2WOff {
  uint32_t base[2], last[2], dummy[2];
  uint32_t block;  // bytes of 16 rows
};
__device__ __forceinline__ void tb2_woff(Tb2WOff& wo, const StreamArgs& a, const Rows& rw, int lane) {
  const uint32_t rowb = uint32_t(a.K) * 2u;
  wo.block = 16u * rowb;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = 8 * h + (lane >> 3);
    const uint32_t part = 16u * uint32_t((lane & 7) ^ (rr & 7));
    wo.base[h] = uint32_t(rw.r0 + rr) * rowb + part;
    wo.last[h] = uint32_t(rw.r1 - 1) * rowb + part;
    wo.dummy[h] = uint32_t(rr) * rowb + part;
  }
}
__device__ __forceinline__ uint32_t tb2_wo(const Tb2WOff& wo, int i, int h) {
  const uint32_t o = wo.base[h] + uint32_t(i) * wo.block;
  return o < wo.last[h] ? o : wo.last[h];
}
__device__ __forceinline__ void tb2_copy_w(char* slot, __amdgpu_buffer_rsrc_t wr, uint32_t o0, uint32_t o1, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)slot, 16, o0, soff, 0, 2);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(slot + 1024), 16, o1, soff, 0, 2);
}
// This wave's 128 tokens at features f .. f + 63 (inside one column): copy k holds tokens
// 16 k .. 16 k + 15, four lanes each, part p of token t at position p ^ ((t >> 2) & 3); then the
// scales of features f .. f + 31 and f + 32 .. f + 63 of every token (the fp32 scale, or the
// aligned dword that holds the E8M0 byte) at 8192 + 512 s + 4 t.  NS = 1 where both halves of
// every chunk share their scale word (fp32 scales per a multiple of 64 features; E8M0 scales,
// whose dwords hold four 32-feature groups): one gather of 64 rows' words fewer per 64 tokens.
// Then, with `fresh` false (the chunk's scale words are those already in the buffer), the scale
// copies are replaced by as many reads of one word into the unused second area, which keeps the
// number of copies per chunk, and with it the wait counts, fixed.
template <int NS>
__device__ __forceinline__ void tb2_copy_tok(char* tbuf, const StreamArgs& a, const int32_t* s_ids, int f, int lane,
                                             bool fresh = true) {
  const int j = f / a.head_dim;
  const int cc = f - j * a.head_dim;
  int rid[10];
#pragma unroll
  for (int k = 0; k < 8; ++k) rid[k] = s_ids[(16 * k + (lane >> 2)) * a.n_cols + j];
#pragma unroll
  for (int k = 0; k < 2; ++k) rid[8 + k] = s_ids[(64 * k + lane) * a.n_cols + j];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int t = 16 * k + (lane >> 2);
    const int64_t rr = rid[k] >= 0 ? rid[k] : 0;
    __builtin_amdgcn_global_load_lds((const void*)(a.table + rr * a.head_dim + cc + 16 * ((lane & 3) ^ ((t >> 2) & 3))),
                                     (lds_ptr_t)(tbuf + k * 1024), 16, 0, 0);
  }
  const int nb = a.head_dim / a.scale_block;
  const int sbyte = a.scale_e8m0 ? 1 : 4;
  if (NS == 1 && !fresh) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
      __builtin_amdgcn_global_load_lds(a.scales, (lds_ptr_t)(tbuf + 8192 + 512 + k * 256), 4, 0, 0);
    return;
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t rr = rid[8 + k] >= 0 ? rid[8 + k] : 0;
      const size_t off = size_t(rr * nb + (cc + 32 * s) / a.scale_block) * sbyte;
      __builtin_amdgcn_global_load_lds((const void*)(static_cast<const char*>(a.scales) + (off & ~size_t(3))),
                                       (lds_ptr_t)(tbuf + 8192 + s * 512 + k * 256), 4, 0, 0);
    }
}

// One chunk's token operands as the lane reads them from its wave's buffer: codes [step][token
// block][sub-block], the scale words, and an all-ones / zero mask per token (ids checked).
struct Tok2Raw {
  u32x2 code[2][2][4];
  uint32_t sw[2][2][4];
  uint32_t keep[2][4];
};

template <int NS>
__device__ __forceinline__ void tb2_read_tok(Tok2Raw& r, const char* my_tok, const int32_t* s_ids, int j,
                                             int n_cols, int lane) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tok = 64 * b + 16 * t + (lane & 15);
      r.keep[b][t] = s_ids[tok * n_cols + j] >= 0 ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int p = 2 * s + (lane >> 5);
        r.code[s][b][t] = *reinterpret_cast<const u32x2*>(my_tok + tok * 64 + 16 * (p ^ ((tok >> 2) & 3)) +
                                                          8 * ((lane >> 4) & 1));
        r.sw[s][b][t] = *reinterpret_cast<const uint32_t*>(my_tok + 8192 + (NS == 2 ? s : 0) * 512 + 4 * tok);
      }
    }
}

// Operand g (step g / 8, token block (g / 4) % 2, sub-block g % 4) of a chunk whose features
// start at cc inside their column.
template <bool E8>
__device__ __forceinline__ void tb2_dequant(u32x4 (&bt)[2][2][4], const Tok2Raw& r, int g, int cc, int scale_block) {
  const int s = g >> 3, b = (g >> 2) & 1, t = g & 3;
  const uint32_t shift8 = uint32_t(((cc + 32 * s) / scale_block) & 3) * 8u;
  const float sc = E8 ? e8m0_to_f32((r.sw[s][b][t] >> shift8) & 0xFFu) : __uint_as_float(r.sw[s][b][t]);
  bt[s][b][t] = masked(dequant8(r.code[s][b][t], sc), r.keep[b][t]);
}

// The K loop.  A wave's weight slots form two stages (NRB x 4 KB of its weights in flight, as
// in the one-block kernel): the slot row block i of chunk c leaves is refilled with chunk c +
// 2's rows right after it is read.  Per chunk the wave first reads and dequantises its token
// operands (which frees its token buffer for chunk c + 1's copies), then multiplies row block
// by row block.
template <int NRB, bool E8, int NS>
__device__ __forceinline__ void tb2_loop(f32x4 (&acc)[2][NRB][4], const StreamArgs& a, const int32_t* s_ids,
                                         char* smem, const Rows& rw, int lane, int wv) {
  // (the wave index as a scalar: the copies' LDS addresses and the chunks' feature offsets are
  // then scalars too, as a buffer copy's scalar offset must be)
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  const int q0 = wvs * (a.K >> 2);
  const int nch = (a.K >> 2) / kC2;
  const int rot = int((5u * blockIdx.x) % uint32_t(nch));
  auto feat = [&](int c) { return q0 + kC2 * ((c + rot) % nch); };
  char* my_slots = smem + wvs * 2 * NRB * kW2Slot;  // stage k: slots k NRB .. k NRB + NRB - 1
  char* my_tok = smem + 8 * NRB * kW2Slot + wvs * kTok2;
  const __amdgpu_buffer_rsrc_t wsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.wkv), (short)0, a.N * a.K * 2, 0x00020000);
  Tb2WOff wo;
  tb2_woff(wo, a, rw, lane);
  // copy order: chunk 0's weights, its tokens, chunk 1's weights; then each chunk c issues chunk
  // c + 1's tokens (kTok copies) and one weight copy per row block (chunk c + 2's).  A chunk's
  // tokens are then always followed by exactly one chunk's weight copies (2 NRB) until they are
  // read, and a row block's copy by the rest of its chunk's, two chunks' tokens, one chunk's
  // weights and as many weight copies as blocks already read: 4 NRB - 2 + 2 kTok copies.
  constexpr int kTok = 8 + 2 * NS;
  // features one scale word covers (NS = 1): a block of fp32 scales, four of E8M0 bytes
  const int span = E8 ? 4 * a.scale_block : a.scale_block;
  const bool two = nch > 1;
#pragma unroll
  for (int i = 0; i < NRB; ++i) {
    tb2_copy_w(my_slots + i * kW2Slot, wsrc, tb2_wo(wo, i, 0), tb2_wo(wo, i, 1), 2 * feat(0));
    asm volatile("" ::: "memory");
  }
  tb2_copy_tok<NS>(my_tok, a, s_ids, feat(0), lane);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < NRB; ++i) {
    if (two) tb2_copy_w(my_slots + (NRB + i) * kW2Slot, wsrc, tb2_wo(wo, i, 0), tb2_wo(wo, i, 1), 2 * feat(1));
    else tb2_copy_w(my_slots + (NRB + i) * kW2Slot, wsrc, wo.dummy[0], wo.dummy[1], 0);
    asm volatile("" ::: "memory");
  }
  constexpr int kInFlight = 4 * NRB - 2 + 2 * kTok;
  static_assert(kInFlight <= 63, "vmcnt range");
  const int wr = lane & 15;
  // one chunk; the stage is a template argument so that the two stages' slot addresses are
  // constants of their own copy of the body
  auto chunk = [&](int c, auto stage_tag) {
    constexpr int st = decltype(stage_tag)::value;
    const int fc = feat(c);
    const int fn = feat(c + 1 < nch ? c + 1 : c);
    const bool live2 = c + 2 < nch;
    const int fnn = feat(live2 ? c + 2 : c);
    char* stage = my_slots + st * NRB * kW2Slot;
    // chunk c's token copies have landed once only chunk c + 1's weight copies remain
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NRB) : "memory");
    u32x4 bt[2][2][4];
    {
      Tok2Raw raw;
      tb2_read_tok<NS>(raw, my_tok, s_ids, fc / a.head_dim, a.n_cols, lane);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the buffer is read before its refill
      const int cc = fc % a.head_dim;
#pragma unroll
      for (int g = 0; g < 16; ++g) tb2_dequant<E8>(bt, raw, g, cc, a.scale_block);
    }
    // (chunk c + 1 reads chunk c's scale words when both lie in one word's span of one column)
    const bool fresh = fn / a.head_dim != fc / a.head_dim || (fn % a.head_dim) / span != (fc % a.head_dim) / span;
    tb2_copy_tok<NS>(my_tok, a, s_ids, fn, lane, fresh);
    asm volatile("" ::: "memory");
    // row block i + 1's fragments are read while block i's MFMAs run (its copy is waited for
    // after the same refills as block i's would be: the count does not change)
    auto read_wf = [&](u32x4 (&wf)[2], int i) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kInFlight) : "memory");
#pragma unroll
      for (int s = 0; s < 2; ++s)
        wf[s] = *reinterpret_cast<const u32x4*>(stage + i * kW2Slot + wr * 128 + 16 * ((4 * s + (lane >> 4)) ^ (wr & 7)));
    };
    auto refill = [&](int i) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot is read before its refill
      if (live2) tb2_copy_w(stage + i * kW2Slot, wsrc, tb2_wo(wo, i, 0), tb2_wo(wo, i, 1), 2 * fnn);
      else tb2_copy_w(stage + i * kW2Slot, wsrc, wo.dummy[0], wo.dummy[1], 0);
      asm volatile("" ::: "memory");
    };
    u32x4 wf[2][2];
    read_wf(wf[0], 0);
    refill(0);
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      if (i + 1 < NRB) read_wf(wf[(i + 1) & 1], i + 1);
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[b][i][t] = mfma16x16x32(wf[i & 1][s], bt[s][b][t], acc[b][i][t]);
      if (i + 1 < NRB) refill(i + 1);
      asm volatile("" ::: "memory");
    }
  };
  for (int c = 0; c < nch; c += 2) {
    chunk(c, std::integral_constant<int, 0>{});
    if (c + 1 < nch) chunk(c + 1, std::integral_constant<int, 1>{});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The last arrivers' part for token blocks bb and bb + 1 (flags last[0], last[1]), with
// barriers that order only the LDS (the slot stores and partial-sum clears need not complete
// before the next block's): for each stream slot this workgroup closed in either block, the partial sums of every contributor of both blocks are loaded in one round
// (in order, as in the one-block epilogue), then each block's gates go to the slots of its apply
// workgroups and its counter and partial sums are cleared.
__device__ __forceinline__ void tb2_gates(const StreamArgs& a, Shared& sh, const Rows& rw, int tid, int bb,
                                          const int (*last)[2]) {
  const int Q = a.N >> 2, G = a.G;
  const int seg_lo = rw.r0 / a.dim;
  const __amdgpu_buffer_rsrc_t wsr = coherent_rsrc(a.ws_hdr);
  const int t = tid & 63, q = tid >> 6;
  const int napb = a.n_apply / a.n_atb;
#pragma unroll 1
  for (int sl = 0; sl < 2; ++sl) {
    const bool L0 = last[0][sl] != 0, L1 = last[1][sl] != 0;
    if (!L0 && !L1) continue;
    const int s = seg_lo + sl;
    const int wf = owner_of_row(s * a.dim, Q, G), wl = owner_of_row((s + 1) * a.dim - 1, Q, G);
    const int nW = wl - wf + 1;
    const int wb0 = wf + (nW * q) / 4, wb1 = wf + (nW * (q + 1)) / 4;
    const int sl_f = row_begin(wf, Q, G) < s * a.dim ? 1 : 0;
    auto poff = [&](int b, int w2) { return partial_off(a, bb + b, w2, w2 == wf ? sl_f : 0) + t * 16; };
    float r[2][3] = {{0.f, 0.f, 0.f}, {0.f, 0.f, 0.f}};
    for (int base = wb0; base < wb1; base += 16) {
      f32x4 v[2][16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int w2 = base + k < wb1 ? base + k : wb0;
        v[0][k] = L0 ? load_coherent4(wsr, poff(0, w2)) : f32x4{0.f, 0.f, 0.f, 0.f};
        v[1][k] = L1 ? load_coherent4(wsr, poff(1, w2)) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (base + k < wb1) {
            r[b][0] += v[b][k].x;
            r[b][1] += v[b][k].y;
            r[b][2] += v[b][k].z;
          }
    }
#pragma unroll 1
    for (int b = 0; b < 2; ++b) {
      if (!(b == 0 ? L0 : L1)) continue;
      lds_barrier();  // sh.red is free again
      sh.red[q][t][0] = r[b][0];
      sh.red[q][t][1] = r[b][1];
      sh.red[q][t][2] = r[b][2];
      lds_barrier();
      if (q == 0) sh.red[0][t][0] = int64_t(bb + b) * kTB + t < a.M ? gate_from_quarters(a, sh, t) : 0.0f;
      lds_barrier();
      if (tid == 0) store_relaxed(counter_of(a, bb + b, s), 0u);
      // apply workgroup ap of the block takes tokens 32 (ap & 1) .. + 31
      for (int i = tid; i < napb * 8; i += 256) {
        const int ap = i >> 3, t4 = 32 * (ap & 1) + 4 * (i & 7);
        store_coherent4(wsr, ws_off(a, apply_slot(a, bb + b, ap, s) + 4 * (i & 7)),
                        __builtin_bit_cast(f32x4, u32x4{__float_as_uint(sh.red[0][t4][0]) | 0x80000000u,
                                                        __float_as_uint(sh.red[0][t4 + 1][0]) | 0x80000000u,
                                                        __float_as_uint(sh.red[0][t4 + 2][0]) | 0x80000000u,
                                                        __float_as_uint(sh.red[0][t4 + 3][0]) | 0x80000000u}));
      }
      for (int w2 = wb0; w2 < wb1; ++w2) store_coherent4(wsr, poff(b, w2), f32x4{0.f, 0.f, 0.f, 0.f});
    }
    lds_barrier();
  }
}

template <int NRB>
__device__ __forceinline__ void tb2_blocks(const StreamArgs& a, char* smem, Shared& sh, int w, const Rows& rw) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* const s_ids = reinterpret_cast<int32_t*>(smem + 8 * NRB * kW2Slot + 4 * kTok2);
  {
    // hash ids of both token blocks, checked once (n_rows < 2^31): -1 marks a row that reads as
    // zeros
    const int n_ids = 2 * kTB * a.n_cols;
    const int64_t n_valid = a.M * a.n_cols;
    for (int base = 0; base < n_ids; base += 8 * 256) {
      int64_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = base + q * 256 + tid;
        v[q] = i < n_valid ? a.hash_ids[i] : -1;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = base + q * 256 + tid;
        int64_t r = v[q];
        if (i < n_valid && (r < 0 || r >= a.n_rows)) {
          if (w == 0 && a.err_count != nullptr) atomicAdd(a.err_count, 1);
          r = -1;
        }
        if (i < n_ids) s_ids[i] = int32_t(r);
      }
    }
    __syncthreads();
  }
  f32x4 acc[2][NRB][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[b][i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // (E8M0 scale dwords hold four 32-feature groups: both halves of a 64-feature chunk in one)
  if (a.scale_e8m0) tb2_loop<NRB, true, 1>(acc, a, s_ids, smem, rw, lane, wv);
  else if (a.scale_block % 64 == 0) tb2_loop<NRB, false, 1>(acc, a, s_ids, smem, rw, lane, wv);
  else tb2_loop<NRB, false, 2>(acc, a, s_ids, smem, rw, lane, wv);
  __syncthreads();
  // Both token blocks' K-partial reductions and key partial sums first (block 0's stores in
  // flight under block 1's reduction), counted in with one drain and one round of atomics; then
  // the last arrivers' gates for both blocks, so that block 1's gates do not wait behind block
  // 0's hand-off; then the value columns.
  KeyPre<NRB> kp[2];
  f32x4 red[2][NRB];
  prefetch_key<NRB>(kp[0], a, rw, 0, tid);
  prefetch_key<NRB>(kp[1], a, rw, kTB, tid);
  reduce_k<NRB, true>(red[0], acc[0], reinterpret_cast<f32x4*>(smem), rw.nblk, lane, wv);
  epilogue<NRB, true, true, false, kPhStore>(a, red[0], kp[0], sh, 0, w, rw, tid, smem);
  reduce_k<NRB, true>(red[1], acc[1], reinterpret_cast<f32x4*>(smem), rw.nblk, lane, wv);
  epilogue<NRB, true, true, false, kPhStore>(a, red[1], kp[1], sh, 1, w, rw, tid, smem);
  {
    const int seg_lo = rw.r0 / a.dim, seg_hi = (rw.r1 - 1) / a.dim;
    drain_memory_ops();
    __syncthreads();
    if (tid == 0) {
      const int Q = a.N >> 2, G = a.G;
      uint32_t old[2][2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const int s = seg_lo + sl;
          old[b][sl] = s <= seg_hi && s < 4 ? atomic_add_relaxed(counter_of(a, b, s), 1u) : 0u;
        }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const int s = seg_lo + sl;
          const int s3 = s < 4 ? s : 3;
          const int wf = owner_of_row(s3 * a.dim, Q, G), wl = owner_of_row((s3 + 1) * a.dim - 1, Q, G);
          sh.last2[b][sl] = s <= seg_hi && s < 4 && old[b][sl] == uint32_t(wl - wf) ? 1 : 0;
        }
    }
    __syncthreads();
  }
  tb2_gates(a, sh, rw, tid, 0, sh.last2);
  // value columns: each block's bf16 values into this workgroup's tile for that block (the
  // apply workgroups write out)
  epilogue<NRB, true, true, true, kPhValue>(a, red[0], kp[0], sh, 0, w, rw, tid, smem);
  epilogue<NRB, true, true, true, kPhValue>(a, red[1], kp[1], sh, 1, w, rw, tid, smem);
}

template <int NLO, int NHI>
__global__ __launch_bounds__(256, 1) void k_stream_tb2(StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  Shared& sh = *reinterpret_cast<Shared*>(smem + kRedBytes);
  static_assert(stage_bytes(NHI) <= NHI * 16384, "output staging exceeds the reduction buffer");
  const int G = a.G, w = blockIdx.x;
  if (w >= G) {
    apply_wg(a, smem, w - G);
    return;
  }
  const Rows rw = rows_of(w, a.N, G);
  if constexpr (NLO == NHI) {
    tb2_blocks<NLO>(a, smem, sh, w, rw);
  } else {
    if (rw.nblk == NLO) tb2_blocks<NLO>(a, smem, sh, w, rw);
    else tb2_blocks<NHI>(a, smem, sh, w, rw);
  }
}

// ------------------------------------------------------------------------------ four token blocks
// The fused forward of 129..256 tokens in one pass over the weights, from the tokens gathered
// and dequantised beforehand (bf16, in the MFMA's operand order, in the staging area).  One
// workgroup per CU over its NRB row blocks, twelve waves in two roles.  Waves 8..11 copy the
// workgroup's weight rows into a ring of D stages of 128 features (NRB 4 KB slots each, the
// one-block kernel's slot layout: 256 bytes of each row) and wait only for their own copies;
// waves 0..7 each multiply 32 tokens over all of K, their token fragments loaded from the staging
// area (an L2-resident 3 MB at 256 tokens) straight into registers kTb4Tok stages ahead.  A
// wave's memory counter thus covers one kind of access: the copies keep D - 1 stages (up to NRB x
// 4 KB each) in flight, independently of the token loads.  One workgroup barrier per stage: the
// copy waves reach it once the stage has landed, the multiplying waves once they have read the
// stage before it, whose slot the copies issued after the barrier refill.  Then the copy waves
// leave (a barrier waits only for the waves still running), the sums go through LDS, waves 4..7
// leave too, and waves 0..3 take the four blocks through the two-token-block kernel's hand-off:
// key partial sums stored, counted in with one round of atomics, the last arrivers' gates, the
// value workgroups' bf16 tiles for the apply workgroups.
constexpr int kTb4Tok = 2;  // stages of token fragments in flight per multiplying wave
// 16-token sub-blocks per multiplying wave: 16 / kTb4NT such waves (eight of 32 tokens, two per
// SIMD, so that one wave's barrier wait and token loads overlap the other's MFMAs)
constexpr int kTb4NT = 2;
constexpr int kC4 = 128;  // features per stage: 256 bytes of each weight row
// A stage: NRB 4 KB slots, or with TRIM (every workgroup's last row block holds four rows) the
// last one a 1 KB slot of its four rows.
__host__ __device__ constexpr int tb4_stage(int nrb, bool trim) { return trim ? (nrb - 1) * kWBlk + 1024 : nrb * kWBlk; }
__host__ __device__ constexpr int tb4_ring(int nrb, bool trim = false) {
  return 163840 / tb4_stage(nrb, trim) < 12 ? 163840 / tb4_stage(nrb, trim) : 12;
}
// after the loop: the four blocks' sums (NRB x 16 KB) behind the epilogue's shared words, where
// they stay while the epilogue runs
constexpr int kTb4X = (kRedBytes + int(sizeof(Shared)) + 4095) & ~4095;
__host__ __device__ constexpr int tb4_lds(int nrb, bool trim = false) {
  return tb4_ring(nrb, trim) * tb4_stage(nrb, trim) > kTb4X + nrb * 16384 ? tb4_ring(nrb, trim) * tb4_stage(nrb, trim)
                                                                         : kTb4X + nrb * 16384;
}

// Copy wave PI: rows 4 PI .. 4 PI + 3 of every row block (NRB copies of 4 rows x 256 bytes per
// stage, through a buffer resource on wkv), lane l at 16 l: row 4 PI + l / 16 of the block,
// position l % 16 holding the 16-byte part (l % 16) ^ row of the row's 256 stage bytes, as the
// one-block kernel's slots.  A lane's byte offset of its row in block 0, and in the workgroup's
// last row (rows past it repeat it), are computed once; the stage's byte offset is a scalar.
// Stages past the last one copy rows 0..15 at feature 0 (cache resident) into the free slot
// instead, so that the count of copies per stage, and with it the wait before each barrier,
// stays fixed.  With TRIM the last block's slot holds only its four rows (copy wave 0's).
template <int NRB, int PI, bool TRIM>
__device__ __forceinline__ void tb4_produce(const StreamArgs& a, char* smem, const Rows& rw, int lane, int nst,
                                            int rot) {
  constexpr int D = tb4_ring(NRB, TRIM);
  constexpr int kStage = tb4_stage(NRB, TRIM);
  // (with TRIM only copy wave 0 has rows in the last block)
  constexpr int NP = TRIM && PI > 0 ? NRB - 1 : NRB;
  static_assert(D >= 3 && (D - 1) * NP <= 63, "copies in flight within the counter's range");
  const __amdgpu_buffer_rsrc_t wsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.wkv), (short)0, a.N * a.K * 2, 0x00020000);
  const uint32_t rowb = uint32_t(a.K) * 2u;
  const int rr = 4 * PI + (lane >> 4);  // the lane's row in its block
  const uint32_t part = 16u * uint32_t((lane & 15) ^ rr);
  const uint32_t base = uint32_t(rw.r0 + rr) * rowb + part;
  const uint32_t last = uint32_t(rw.r1 - 1) * rowb + part;
  const uint32_t dummy = uint32_t(rr) * rowb + part;
  auto issue = [&](int c, char* slot) {
    const bool live = c < nst;
    const int soff = live ? 2 * kC4 * ((c + rot) % nst) : 0;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const uint32_t oi = base + uint32_t(i) * 16u * rowb;
      const uint32_t o = live ? (oi < last ? oi : last) : dummy;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrc, (lds_ptr_t)(slot + i * kWBlk + PI * 1024), 16, o, soff, 0, 2);
    }
    asm volatile("" ::: "memory");
  };
#pragma unroll 1
  for (int c = 0; c < D - 1; ++c) issue(c, smem + c * kStage);
  char* nslot = smem + (D - 1) * kStage;  // the slot of stage c + D - 1
#pragma unroll 1
  for (int c = 0; c < nst; ++c) {
    // stage c has landed once only the D - 2 stages after it remain
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((D - 2) * NP) : "memory");
    issue(c + D - 1, nslot);
    nslot = nslot + kStage == smem + D * kStage ? smem : nslot + kStage;
  }
  // every copy has landed before the multiplying waves reuse the LDS
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

// Multiplying wave cb: token block cb over all of K, stage by stage from the ring.  The tokens
// are staged in the MFMA's operand order (1 KB per 16 tokens x 32 features, lane l's 16 bytes at
// 16 l: token l % 16, features 8 (l / 16) ..), so that every load reads 1 KB in one run; the rows
// past the last token up to a multiple of 16 are staged as zeros, the sub-blocks after them read
// as zeros through the buffer resource's range.
template <int NRB, int NT, bool TRIM>
__device__ __forceinline__ void tb4_consume(f32x4 (&acc)[NRB][NT], const StreamArgs& a, const char* smem, int lane,
                                            int cw, int nst, int rot) {
  constexpr int D = tb4_ring(NRB, TRIM);
  constexpr int kStage = tb4_stage(NRB, TRIM);
  constexpr int P = kTb4Tok;
  const __amdgpu_buffer_rsrc_t tsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.emb), (short)0, int((a.M + 15) & ~int64_t(15)) * a.K * 2, 0x00020000);
  // the wave's sub-block t (16 tokens): group NT cw + t, its 1 KB blocks at (NT cw + t) x K / 32
  // + k32
  uint32_t vo[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) vo[t] = uint32_t(NT * cw + t) * uint32_t(a.K / 32) * 1024u + 16u * uint32_t(lane);
  u32x4 tk[P][4][NT];
  auto load = [&](u32x4 (&dst)[4][NT], int c) {
    const uint32_t fb = 4096u * uint32_t((c < nst ? c + rot : rot) % nst);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        dst[s][t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(tsrc, vo[t] + fb + 1024u * s, 0, 0));
  };
  // (in stage order, as the loop issues them: otherwise the loads pending at the top of the loop
  // differ in order between its entry and its back edge, and the compiler waits for all of them)
#pragma unroll
  for (int r = 0; r < P; ++r) {
    load(tk[r], r);
    asm volatile("" ::: "memory");
  }
  const int wr = lane & 15;
  const char* slot = smem;
  auto stage = [&](int c, auto reg_tag) {
    constexpr int r = decltype(reg_tag)::value;
    // stage c has landed; this wave's reads of stage c - 1 are done
    lds_barrier();
    // row block i + 1's fragments are read while block i's MFMAs run (K step s, lane group g:
    // part 4 s + g of the row, at position (4 s + g) ^ row)
    // (with TRIM the last block's lanes of rows 4..15 read row 3: their sums are never used)
    u32x4 wf[2][4];
    auto read_wf = [&](u32x4 (&f)[4], int i) {
      const int lr = TRIM && i == NRB - 1 ? (wr < 3 ? wr : 3) : wr;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        f[s] = *reinterpret_cast<const u32x4*>(slot + i * kWBlk + lr * 256 + 16 * ((4 * s + (lane >> 4)) ^ lr));
    };
    read_wf(wf[0], 0);
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      if (i + 1 < NRB) read_wf(wf[(i + 1) & 1], i + 1);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = mfma16x16x32(wf[i & 1][s], tk[r][s][t], acc[i][t]);
    }
    load(tk[r], c + P);
    slot = slot + kStage == smem + D * kStage ? smem : slot + kStage;
  };
  // (nst is even, so that every pass through the loop takes both halves: with a branch around
  // the second half the compiler would wait for every token load at the top of the loop)
  static_assert(P == 2, "the stage body is unrolled by two");
  for (int c = 0; c < nst; c += 2) {
    stage(c, std::integral_constant<int, 0>{});
    stage(c + 1, std::integral_constant<int, 1>{});
  }
  // the copy waves' last copies have landed
  lds_barrier();
}

// The multiplying waves' sums after the loop: X[((b NRB + i) 4 + t) 64 + lane] holds row block i
// of token sub-block t of block b (written by every multiplying wave, then read by waves 0..3:
// wave wv takes sub-block wv of each block, as after the K-partial reduction of the other
// kernels).
template <int NRB>
__device__ __forceinline__ void tb4_blocks(const StreamArgs& a, char* smem, Shared& sh, int w, const Rows& rw) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_tb = int((a.M + kTB - 1) / kTB);
  const f32x4* const X = reinterpret_cast<const f32x4*>(smem + kTb4X);
  auto red_of = [&](f32x4 (&r)[NRB], int b) {
#pragma unroll
    for (int i = 0; i < NRB; ++i) r[i] = X[((b * NRB + i) * 4 + wv) * 64 + lane];
  };
  // the key columns' partial sums of every block (every block's inputs loaded at once: one
  // memory round trip; the products q k, the same for every block, loaded once)
  KeyPre<NRB> kp[4];
  prefetch_key<NRB>(kp[0], a, rw, 0, tid);
#pragma unroll
  for (int b = 1; b < 4; ++b)
    if (b < n_tb) prefetch_key_x<NRB>(kp[b], a, rw, int64_t(b) * kTB, tid, kp[0]);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b < n_tb) {
      f32x4 red[NRB];
      red_of(red, b);
      epilogue<NRB, true, true, false, kPhStore>(a, red, kp[b], sh, b, w, rw, tid, smem);
    }
  }
  // counted in for every block with one drain and one round of atomics
  {
    const int seg_lo = rw.r0 / a.dim, seg_hi = (rw.r1 - 1) / a.dim;
    drain_memory_ops();
    __syncthreads();
    if (tid == 0) {
      const int Q = a.N >> 2, G = a.G;
      uint32_t old[4][2];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const int s = seg_lo + sl;
          old[b][sl] = b < n_tb && s <= seg_hi && s < 4 ? atomic_add_relaxed(counter_of(a, b, s), 1u) : 0u;
        }
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const int s = seg_lo + sl;
          const int s3 = s < 4 ? s : 3;
          const int wf = owner_of_row(s3 * a.dim, Q, G), wl = owner_of_row((s3 + 1) * a.dim - 1, Q, G);
          sh.last4[b][sl] = b < n_tb && s <= seg_hi && s < 4 && old[b][sl] == uint32_t(wl - wf) ? 1 : 0;
        }
    }
    __syncthreads();
  }
  // the last arrivers' gates, two blocks per round (a stream's last arriver is mostly the same
  // workgroup in every block)
  tb2_gates(a, sh, rw, tid, 0, sh.last4);
  tb2_gates(a, sh, rw, tid, 2, sh.last4 + 2);
  // the value columns: each block's bf16 values into this workgroup's tile for that block (one
  // copy of the code for every block: it runs once per call, cold in the instruction cache)
#pragma unroll 1
  for (int b = 0; b < n_tb; ++b) {
    f32x4 red[NRB];
    red_of(red, b);
    epilogue<NRB, true, true, true, kPhValue | kPhNoMark>(a, red, kp[0], sh, b, w, rw, tid, smem);
  }
  // every block's tile stored, then their ready marks (one drain for all blocks)
  if ((rw.r1 - 1) / a.dim == 4) {
    drain_memory_ops();
    __syncthreads();
    const int j = w - owner_of_row(4 * a.dim, a.N >> 2, a.G);
    if (tid < 2 * n_tb) store_relaxed(apply_slot(a, tid >> 1, 2 * j + (tid & 1), 4), 0x80000000u);
  }
}

template <int NRB, int NT, bool TRIM>
__global__ __launch_bounds__((16 / NT + 4) * 64, 1) void k_stream_tb4(StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  Shared& sh = *reinterpret_cast<Shared*>(smem + kRedBytes);
  const int G = a.G, w = blockIdx.x;
  // (the wave index as a scalar: a role is taken by whole waves, and the copies' LDS addresses
  // and feature offsets are scalars)
  const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= G) {
    // apply workgroups: four waves, as in the other fused kernels; the rest leave at once
    if (wv < 4) apply_wg(a, smem, w - G);
    return;
  }
  const Rows rw = rows_of(w, a.N, G);
  const int nst = a.K / kC4;
  const int rot = int((5u * uint32_t(w)) % uint32_t(nst));
  // waves 0 .. NC - 1 multiply (NT sub-blocks of 16 tokens each), the next four copy
  constexpr int NC = 16 / NT;
  if (wv >= NC) {
    const int p = wv - NC;
    if (p == 0) tb4_produce<NRB, 0, TRIM>(a, smem, rw, lane, nst, rot);
    else if (p == 1) tb4_produce<NRB, 1, TRIM>(a, smem, rw, lane, nst, rot);
    else if (p == 2) tb4_produce<NRB, 2, TRIM>(a, smem, rw, lane, nst, rot);
    else tb4_produce<NRB, 3, TRIM>(a, smem, rw, lane, nst, rot);
    return;
  }
  f32x4 acc[NRB][NT];
#pragma unroll
  for (int i = 0; i < NRB; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  tb4_consume<NRB, NT, TRIM>(acc, a, smem, lane, wv, nst, rot);
  {
    // the sums through LDS (sub-block g = NT wv + t: block g / 4, sub-block g % 4)
    f32x4* const X = reinterpret_cast<f32x4*>(smem + kTb4X);
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int g = NT * wv + t;
        X[(((g >> 2) * NRB + i) * 4 + (g & 3)) * 64 + lane] = acc[i][t];
      }
    lds_barrier();
  }
  // the epilogue takes four waves; the other multiplying waves leave
  if (wv >= 4) return;
  tb4_blocks<NRB>(a, smem, sh, w, rw);
}

template <bool FUSED, int NRB>
void* pick_narrow(int nstep) {
  if (nstep % 3 == 0) return reinterpret_cast<void*>(&k_stream_narrow<NRB, 3, FUSED>);
  if (nstep % 2 == 0) return reinterpret_cast<void*>(&k_stream_narrow<NRB, 2, FUSED>);
  return reinterpret_cast<void*>(&k_stream_narrow<NRB, 1, FUSED>);
}

// With MXFP8 weights the fused kernel runs a single token block (larger calls expand the
// weights and take a bf16 schedule) and the projection alone always loops over token blocks,
// which halves the instantiations.
template <int NLO, bool FUSED, bool W8, bool MX>
void* pick_wide_n(bool same, bool one_tb) {
  if constexpr (W8) one_tb = FUSED;
  if (one_tb) {
    if constexpr (W8 && !FUSED) return nullptr;
    else
      return same ? reinterpret_cast<void*>(&k_stream_wide<NLO, NLO, FUSED, true, W8, MX>)
                  : reinterpret_cast<void*>(&k_stream_wide<NLO, NLO + 1, FUSED, true, W8, MX>);
  }
  if constexpr (MX) return nullptr;
  if constexpr (W8 && FUSED) return nullptr;
  else
    return same ? reinterpret_cast<void*>(&k_stream_wide<NLO, NLO, FUSED, false, W8>)
                : reinterpret_cast<void*>(&k_stream_wide<NLO, NLO + 1, FUSED, false, W8>);
}

// The deep decode loop: one row-block count NRB, the last block four rows.
template <int NRB>
void* pick_deep_n() {
  return reinterpret_cast<void*>(&k_stream_wide<NRB, NRB, true, true, false, false, true>);
}
void* pick_deep(int nrb) {
  switch (nrb) {
    case 2: return pick_deep_n<2>();
    case 3: return pick_deep_n<3>();
    case 4: return pick_deep_n<4>();
    case 5: return pick_deep_n<5>();
    case 6: return pick_deep_n<6>();
    case 7: return pick_deep_n<7>();
    default: return nullptr;
  }
}

template <bool FUSED, bool W8, bool MX = false>
void* pick_wide(int nlo, int nhi, bool one_tb) {
  const bool same = nlo == nhi;
  switch (nlo) {
    case 1: return pick_wide_n<1, FUSED, W8, MX>(same, one_tb);
    case 2: return pick_wide_n<2, FUSED, W8, MX>(same, one_tb);
    case 3: return pick_wide_n<3, FUSED, W8, MX>(same, one_tb);
    case 4: return pick_wide_n<4, FUSED, W8, MX>(same, one_tb);
    case 5: return pick_wide_n<5, FUSED, W8, MX>(same, one_tb);
    case 6: return pick_wide_n<6, FUSED, W8, MX>(same, one_tb);
    case 7: return pick_wide_n<7, FUSED, W8, MX>(same, one_tb);
    default: return nullptr;
  }
}

// Workgroups that own a value row (the owner of the first value row, 4 dim, and all after it).
int value_groups(int N, int dim, int G) {
  const int Q = N / 4;
  const int v0 = int((uint32_t((4 * dim) / 4 + 1) * uint32_t(G) - 1u) / uint32_t(Q));
  return G - v0;
}

// Fewest and most 16-row blocks of a workgroup (rows per workgroup: 4 floor(Q / G) or
// 4 ceil(Q / G)).
int min_blocks(int N, int G) { return (4 * ((N / 4) / G) + 15) / 16; }
int max_blocks(int N, int G) { return (4 * ((N / 4 + G - 1) / G) + 15) / 16; }

bool use_wide(const StreamArgs& a, int G, bool fused) {
  // a 128-feature chunk stays in one column and a lane's 32 features share one scale
  const bool hd_ok = !fused || (a.head_dim % 128 == 0 && a.scale_block % 32 == 0);
  const int lo = min_blocks(a.N, G), hi = max_blocks(a.N, G);
  return (a.K / 4) % 128 == 0 && hd_ok && lo >= 1 && lo <= 7 && hi <= lo + 1;
}

// LDS of a launch: the wide loop's slots and buffers (or the narrow loop's reduction buffer), the
// staged hash ids, and with MXFP8 weights the weight-scale table and (scaled fp8 MFMA) the
// waves' token-scale tables.
size_t stream_lds(int N, int K, int n_cols, int head_dim, int scale_block, int G, bool fused, bool wide, bool w8,
                  bool mx) {
  size_t lds = size_t(wide ? wide_lds_bytes(max_blocks(N, G), fused, w8) : kRedBytes) +
               (fused ? size_t(kTB) * n_cols * 8 : 0);
  if (w8) lds += (size_t(stream_rows_per_group(N, G)) * (K / 32) + 15) & ~size_t(15);
  if (mx) lds += 4 * size_t(kTB) * ((K / 4) / head_dim) * (head_dim / scale_block);
  if (lds < kRedBytes + sizeof(Shared)) lds = kRedBytes + sizeof(Shared);
  return lds;
}

// The scaled fp8 MFMA in the fused kernel: an MXFP8 table whose rows' scales for a wave's K
// quarter form whole columns, and LDS for the token-scale tables.
bool stream_mx_ok(const StreamArgs& a, int G) {
  return a.scale_e8m0 && (a.K / 4) % a.head_dim == 0 &&
         stream_lds(a.N, a.K, a.n_cols, a.head_dim, a.scale_block, G, true, true, true, true) <= 163840;
}

// Dynamic LDS above the default 64 KB: raise the kernel's limit once (a kernel's need is fixed
// by its shape class, and the largest value set so far stays in force).
hipError_t allow_lds(void* fn, size_t lds) {
  if (lds > 163840) return hipErrorInvalidValue;
  if (lds <= 65536) return hipSuccess;
  static std::mutex mu;
  static void* raised[64];
  static int raised_lds[64];
  static int n_raised = 0;
  std::lock_guard<std::mutex> lock(mu);
  int k = 0;
  while (k < n_raised && raised[k] != fn) ++k;
  if (k == n_raised || raised_lds[k] < int(lds)) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    if (k == n_raised && n_raised < 64) {
      raised[n_raised] = fn;
      raised_lds[n_raised++] = int(lds);
    } else if (k < n_raised) {
      raised_lds[k] = int(lds);
    }
  }
  return hipSuccess;
}

template <bool FUSED>
hipError_t launch_stream_impl(const StreamArgs& a, int G, hipStream_t stream) {
  void* fn = nullptr;
  const bool wide = use_wide(a, G, FUSED);
  bool mx = false, deep = false;
  if (a.w8) {
    // MXFP8 weights: the wide loop only; the fused kernel takes one token block
    if (!wide || (FUSED && a.M > kTB)) return hipErrorInvalidValue;
    // an MXFP8 table too: both operands stay fp8 (the scaled MFMA)
    mx = FUSED && stream_mx_ok(a, G);
    if (mx) fn = pick_wide<true, true, true>(min_blocks(a.N, G), max_blocks(a.N, G), true);
    else fn = pick_wide<FUSED, true>(min_blocks(a.N, G), max_blocks(a.N, G), a.M <= kTB);
  } else if (wide) {
    fn = pick_wide<FUSED, false>(min_blocks(a.N, G), max_blocks(a.N, G), a.M <= kTB);
    // one token block where every workgroup's rows end in a four-row block: the deep loop
    const int rows = stream_rows_per_group(a.N, G), nrb = max_blocks(a.N, G);
    if (FUSED && a.M <= kTB && (a.N / 4) % G == 0 && rows % 16 == 4 && nrb >= 2 && a.n_rows <= 0x7FFFFFFF &&
        size_t(deep_lds_bytes(nrb, a.n_cols)) <= 163840 && pick_deep(nrb) != nullptr) {
      fn = pick_deep(nrb);
      deep = true;
    }
  } else {
    const int per_wg = max_blocks(a.N, G);
    const int nstep = (a.K / 4) / 32;
    if (per_wg <= 1) fn = pick_narrow<FUSED, 1>(nstep);
    else if (per_wg <= 2) fn = pick_narrow<FUSED, 2>(nstep);
    else if (per_wg <= 4) fn = pick_narrow<FUSED, 4>(nstep);
    else if (per_wg <= 8) fn = pick_narrow<FUSED, 8>(nstep);
  }
  if (fn == nullptr) return hipErrorInvalidValue;
  StreamArgs arg = a;
  arg.G = G;
  arg.n_apply = 0;
  arg.n_atb = 0;
  if (FUSED && wide && (a.w8 || a.M <= kTB)) {
    // the one-token-block fused kernel: two apply workgroups per value workgroup, whose slots
    // (5 x 32 words each) fit in the token block's gate-slot region (G x 4 x 64 words)
    const int V = value_groups(a.N, a.dim, G);
    if (V < 1 || 2 * V * 160 > G * 256) return hipErrorInvalidValue;
    arg.n_apply = 2 * V;
    arg.n_atb = 1;
  }
  void* params[] = {&arg};
  size_t lds = stream_lds(a.N, a.K, a.n_cols, a.head_dim, a.scale_block, G, FUSED, wide, a.w8 != 0, mx);
  if (deep) {
    lds = size_t(deep_lds_bytes(max_blocks(a.N, G), a.n_cols));
    if (lds < kRedBytes + sizeof(Shared)) lds = kRedBytes + sizeof(Shared);
  }
  const hipError_t e = allow_lds(fn, lds);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(fn, dim3(G + arg.n_apply), dim3(256), params, lds, stream);
}

template <int NLO>
void* pick_tb2_n(bool same) {
  return same ? reinterpret_cast<void*>(&k_stream_tb2<NLO, NLO>)
              : reinterpret_cast<void*>(&k_stream_tb2<NLO, (NLO < 7 ? NLO + 1 : 7)>);
}
void* pick_tb2(int nlo, int nhi) {
  const bool same = nlo == nhi;
  if (!same && (nhi != nlo + 1 || nhi > 7)) return nullptr;
  switch (nlo) {
    case 1: return pick_tb2_n<1>(same);
    case 2: return pick_tb2_n<2>(same);
    case 3: return pick_tb2_n<3>(same);
    case 4: return pick_tb2_n<4>(same);
    case 5: return pick_tb2_n<5>(same);
    case 6: return pick_tb2_n<6>(same);
    case 7: return same ? pick_tb2_n<7>(true) : nullptr;
    default: return nullptr;
  }
}


}  // namespace

int stream_grid(int N, int num_cus) {
  const int Q = N / 4;
  int G = num_cus;
  if (G > Q) G = Q;
  while (max_blocks(N, G) > 8) ++G;  // at most 8 row blocks per workgroup
  return G;
}

int stream_rows_per_group(int N, int G) { return 4 * ((N / 4 + G - 1) / G); }

bool stream_w8_ok(int K, int N, int head_dim, int scale_block, int num_cus, bool fused) {
  StreamArgs a;
  memset(&a, 0, sizeof(a));
  a.K = K;
  a.N = N;
  a.head_dim = head_dim;
  a.scale_block = scale_block;
  const int G = stream_grid(N, num_cus);
  if (!use_wide(a, G, fused)) return false;
  // weight slots, token buffers, staged ids and the scale table fit in the LDS
  return stream_lds(N, K, K / head_dim, head_dim, scale_block, G, fused, true, true, false) <= 163840;
}

// Workspace: a 256-byte header (word 0 counts wait time-outs), then one block per 64-token
// block at a fixed stride that depends only on the grid.
size_t stream_tb_stride(int grid) {
  return size_t(256) * 4 + size_t(grid) * 4 * kTB * 4 + size_t(grid) * 2 * kTB * 16;
}

// The fused forward of one to four token blocks also needs the blocks' value tiles behind their
// control words (cleared again by the apply workgroups); the larger of the two layouts, so that
// the size never decreases with M.
size_t stream_workspace_bytes(int64_t M, int N, int dim, int grid) {
  const int64_t n_tb = (M + kTB - 1) / kTB;
  const size_t blocks = size_t(n_tb) * stream_tb_stride(grid);
  const int64_t n_atb = n_tb < 4 ? (n_tb < 1 ? 1 : n_tb) : 4;
  const size_t tiled = size_t(n_atb) * (stream_tb_stride(grid) + size_t(value_groups(N, dim, grid)) * kVTile);
  return 256 + (blocks > tiled ? blocks : tiled);
}

hipError_t launch_kv_proj_stream(const StreamArgs& a, int num_cus, hipStream_t stream) {
  return launch_stream_impl<false>(a, stream_grid(a.N, num_cus), stream);
}

// The two-token-block kernel (65..128 tokens): bf16 weights of at most 2^31 - 1 bytes (copied
// through a buffer resource); 64-feature chunks inside one table column (head_dim a multiple of
// 64) and 32-feature groups inside one scale block; one or two row-block counts per workgroup,
// at most seven; its LDS within the CU's; the apply workgroups' slots within each token
// block's gate-slot region.
bool stream_tb2_ok(int K, int N, int dim, int n_cols, int head_dim, int scale_block, int num_cus) {
  const int G = stream_grid(N, num_cus);
  const int lo = min_blocks(N, G), hi = max_blocks(N, G);
  const int V = value_groups(N, dim, G);
  return (K / 4) % kC2 == 0 && head_dim % kC2 == 0 && scale_block % 32 == 0 && lo >= 1 && hi <= 7 &&
         hi <= lo + 1 && tb2_lds(hi, n_cols) <= 163840 && int64_t(N) * K * 2 <= 0x7FFFFFFF &&
         V >= 1 && 2 * V * 160 <= G * 256;
}

hipError_t launch_forward_tb2(StreamArgs a, void* workspace, int num_cus, hipStream_t stream) {
  if (a.M <= kTB || a.M > 2 * kTB || a.w8 || a.n_rows > 0x7FFFFFFF ||
      !stream_tb2_ok(a.K, a.N, a.dim, a.n_cols, a.head_dim, a.scale_block, num_cus))
    return hipErrorInvalidValue;
  const int G = stream_grid(a.N, num_cus);
  a.ws_hdr = static_cast<uint32_t*>(workspace);
  a.tb_stride = stream_tb_stride(G);
  a.G = G;
  // two apply workgroups per value workgroup and token block, their slots (5 x 32 words each)
  // in the block's gate-slot region (G x 4 x 64 words)
  a.n_atb = 2;
  a.n_apply = 4 * value_groups(a.N, a.dim, G);
  void* fn = pick_tb2(min_blocks(a.N, G), max_blocks(a.N, G));
  if (fn == nullptr) return hipErrorInvalidValue;
  const size_t lds = size_t(tb2_lds(max_blocks(a.N, G), a.n_cols));
  const hipError_t e = allow_lds(fn, lds);
  if (e != hipSuccess) return e;
  void* params[] = {&a};
  return hipLaunchKernel(fn, dim3(G + a.n_apply), dim3(256), params, lds, stream);
}

// The four-token-block kernel (129..256 tokens from staged bf16 rows): every workgroup owns the
// same number of row blocks, at most seven; an even number of 128-feature stages; bf16 weights and staged tokens of
// at most 2^31 - 1 bytes each (read through buffer resources); the apply workgroups' slots within
// each token block's gate-slot region.
bool stream_tb4_ok(int K, int N, int dim, int num_cus) {
  const int G = stream_grid(N, num_cus);
  const int lo = min_blocks(N, G), hi = max_blocks(N, G);
  const int V = value_groups(N, dim, G);
  const bool trim = hi >= 2 && stream_rows_per_group(N, G) % 16 == 4;
  return (N / 4) % G == 0 && K % (2 * kC4) == 0 && lo == hi && hi >= 1 && hi <= 7 && tb4_lds(hi, trim) <= 163840 &&
         int64_t(N) * K * 2 <= 0x7FFFFFFF && int64_t(4 * kTB) * K * 2 <= 0x7FFFFFFF && V >= 1 &&
         2 * V * 160 <= G * 256;
}

template <bool TRIM>
void* pick_tb4(int nrb) {
  switch (nrb) {
    case 1: return TRIM ? nullptr : reinterpret_cast<void*>(&k_stream_tb4<1, kTb4NT, false>);
    case 2: return reinterpret_cast<void*>(&k_stream_tb4<2, kTb4NT, TRIM>);
    case 3: return reinterpret_cast<void*>(&k_stream_tb4<3, kTb4NT, TRIM>);
    case 4: return reinterpret_cast<void*>(&k_stream_tb4<4, kTb4NT, TRIM>);
    case 5: return reinterpret_cast<void*>(&k_stream_tb4<5, kTb4NT, TRIM>);
    case 6: return reinterpret_cast<void*>(&k_stream_tb4<6, kTb4NT, TRIM>);
    case 7: return reinterpret_cast<void*>(&k_stream_tb4<7, kTb4NT, TRIM>);
    default: return nullptr;
  }
}

hipError_t launch_forward_tb4(StreamArgs a, void* workspace, int num_cus, hipStream_t stream) {
  if (a.M <= 2 * kTB || a.M > 4 * kTB || a.w8 || a.emb == nullptr || !stream_tb4_ok(a.K, a.N, a.dim, num_cus))
    return hipErrorInvalidValue;
  const int G = stream_grid(a.N, num_cus);
  a.ws_hdr = static_cast<uint32_t*>(workspace);
  a.tb_stride = stream_tb_stride(G);
  a.G = G;
  // two apply workgroups per value workgroup and token block
  a.n_atb = int((a.M + kTB - 1) / kTB);
  a.n_apply = 2 * a.n_atb * value_groups(a.N, a.dim, G);
  // the last row block of four rows (every workgroup alike): its slot trimmed to them
  const int nrb = max_blocks(a.N, G);
  const bool trim = nrb >= 2 && stream_rows_per_group(a.N, G) % 16 == 4;
  void* fn = trim ? pick_tb4<true>(nrb) : pick_tb4<false>(nrb);
  if (fn == nullptr) return hipErrorInvalidValue;
  size_t lds = size_t(tb4_lds(nrb, trim));
  if (lds < kRedBytes + sizeof(Shared)) lds = kRedBytes + sizeof(Shared);
  const hipError_t e = allow_lds(fn, lds);
  if (e != hipSuccess) return e;
  void* params[] = {&a};
  return hipLaunchKernel(fn, dim3(G + a.n_apply), dim3((16 / kTb4NT + 4) * 64), params, lds, stream);
}

hipError_t launch_forward_stream(StreamArgs a, void* workspace, int num_cus, hipStream_t stream) {
  const int G = stream_grid(a.N, num_cus);
  a.ws_hdr = static_cast<uint32_t*>(workspace);
  a.tb_stride = stream_tb_stride(G);
  return launch_stream_impl<true>(a, G, stream);
}

}  // namespace engram
