// Tiled wkv projection for large token counts (prefill), alone or fused with the per-stream
// gate and the residual add.  The dequantised rows come from a gather pass that writes them, as
// bf16, into a staging area (k_gather_dequant): at these token counts every row feeds all
// (hc + 1) * dim / 256 column tiles of its token block, and one bf16 write per row costs less
// than re-gathering the fp8 row for every tile.
//
// A workgroup computes one tile of 256 tokens x 256 wkv rows (output columns) over all of K, in
// stages of 64 features.  A stage of one operand is 256 rows of 128 bytes in LDS, 16-byte chunk c
// of row r at position c ^ (r & 7) (conflict-free for the fragment reads below).  wkv stages
// live in a ring of three slots and are copied two stages ahead, token stages in a ring of two,
// copied one stage ahead (5 x 32 KB = 160 KB); every copy is a global -> LDS
// global_load_lds_dwordx4 filling 8 rows x 128 bytes.
//
// Eight waves, two per SIMD.  Waves 0-3 (group 0) own wkv rows 0-127 of the tile, waves 4-7
// (group 1) rows 128-255; within a group, wave w & 3 owns tokens 64 (w & 3) .. + 63.  Each wave
// computes 128 columns x 64 tokens as 8 x 4 blocks of v_mfma_f32_16x16x32_bf16 (128 accumulator
// registers).  The groups alternate ("ping-pong"): while the group-0 wave of a SIMD issues the
// 32 MFMAs of one half stage, the group-1 wave reads its fragments (and issues copies), then the
// roles swap; a workgroup barrier separates phases.  So each SIMD's matrix unit is fed by one
// wave at a time whose operands are already in registers, and the LDS and memory latency of one
// wave hides under the other's MFMAs.  The phase-by-phase schedule and its wait counts are
// spelled out at k_loop.
//
// Split K: when a call has at most 128 tiles (up to 256 tokens at the decode layout), two
// workgroups compute each tile, one over each half of K; the first to finish leaves its fp32
// partial tile in the staging area and the second adds it and runs the epilogue (split_merge).
// With more tiles (bf16 schedule), the tiles of a last, partial round of the grid (tiles mod
// CUs, when at most 128 and at most half the CUs) are split the same way: that round then takes
// half a tile's time on twice as many CUs (3200 tiles at 8192 tokens: 12 full rounds, then 128
// tiles as 256 halves).
//
// fp8 schedule (MXFP8 weights and an MXFP8 table, fused forward only): the gather pass stages
// the rows as fp8 codes plus one E8M0 byte per 32 features, and both operands stay fp8.  A stage
// is 128 features (128-byte rows, the same LDS row layout and copy instructions) plus each row's
// dword of four scales; both operands have rings of two slots (4 x 32 KB + 4 KB of scales), each
// part of a stage copied as soon as its slot's last reader is done (see k_loop_mx).  The MFMA is v_mfma_scale_f32_16x16x128_f8f6f4 (twice the bf16 rate; a
// lane supplies 16-byte parts l / 16 and l / 16 + 4 of its row and the scale of 32-feature block
// l / 16); a half stage is 4 wkv row blocks x 4 token blocks (16 MFMAs of K = 128, as long as the
// 32 bf16 MFMAs of a bf16 half stage), the token fragments being read once per stage.
//
// Tile order: token blocks are taken in groups of 32; inside a group, workgroup b takes token
// block b % 32 and column block b / 32 (a last, smaller group likewise with its own size), so
// the 256 tiles resident at one time cover 32 token panels and 8 weight panels, each XCD
// holding 4 of the one and 8 of the other (the fewest panels per XCD for 32 tiles), and
// (workgroups being dealt to the 8 XCDs round robin) all tiles of a token block run on one
// XCD when its group size is a multiple of 8, keeping its staged rows and its x in that XCD's
// L2.  In the fused kernel every key column block of a token block comes before every value
// column block.  Key tiles post per-(token, stream)
// partial sums of the gate's three reductions; the last key tile of each (token block, stream)
// sums them in column-block order, evaluates the gates and hands them to the value tiles of the
// token block through per-tile slots.  A value tile waits only on key tiles with lower ids,
// which never wait, and every wait is bounded (time-outs are counted in workspace word 0).
#include "common.h"
#include "launch.h"

namespace engram {

namespace {

constexpr int kThreads = 512;               // 8 waves
constexpr int kGroupTb = 32;                // token blocks per tile group
constexpr int kTM = 256;                    // tokens per tile
constexpr int kTN = 256;                    // wkv rows per tile
constexpr int kTK = 64;                     // features per stage
constexpr int kRowB = kTK * 2;              // bytes per LDS row: 8 chunks of 16 bytes
constexpr int kOpB = 256 * kRowB;           // one operand of one stage (32 KB)
constexpr int kARing = 3;                   // wkv stages in LDS
constexpr int kBRing = 2;                   // token stages in LDS
constexpr int kBOff = kARing * kOpB;        // token ring offset
constexpr int kLds = (kARing + kBRing) * kOpB;  // 160 KB, all of a CU's LDS
constexpr int kCopies = 4;                  // copy instructions per wave per operand and stage
constexpr int kBI = 8;                      // 16-column blocks per wave
constexpr int kBJ = 4;                      // 16-token blocks per wave
constexpr int64_t kSplitMaxTiles = 128;     // most tiles split over K in one call

typedef f32x4 TileAcc[kBI][kBJ];
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Everything a wave needs to copy and read stages.
struct Pipe {
  const char* a_src[kCopies];  // per-lane global source of each wkv copy at feature 0
  const char* b_src[kCopies];  // the same for the token copies
  uint32_t frag_off[2];        // per-lane byte offset of a fragment read (stage half 0, 1)
  int wv_u;                    // wave index (wave-uniform)
  int a_off, b_off;            // byte offsets of this wave's first wkv row and first token row
};

// This wave's copies of one operand of stage t into `dst` (one ring slot): row groups
// 4 w .. 4 w + 3 of 8 rows.  Instruction g fills LDS bytes [1024 g, 1024 g + 1024) of the
// slot, lane l at 16 l: row 8 g + (l >> 3), position l & 7, which holds chunk
// (l & 7) ^ (l >> 3), i.e. row r keeps chunk c at position c ^ (r & 7).
__device__ __forceinline__ void copy_op(const char* const (&src)[kCopies], char* dst, int wv_u, int t) {
  const size_t k_bytes = size_t(t) * (kTK * 2);
#pragma unroll
  for (int i = 0; i < kCopies; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(src[i] + k_bytes), (lds_ptr_t)(dst + (4 * wv_u + i) * 1024), 16,
                                     0, 0);
}

// The 12 fragments of one half (32 features) of a stage for this wave: F[i] = wkv rows
// 16 i .. 16 i + 15 of the wave's 128, F[8 + j] = tokens 16 j .. 16 j + 15 of its 64.  Lane l
// gets row l & 15, features 32 hh + 8 (l >> 4) .. + 7 of the stage (the MFMA operand layout).
__device__ __forceinline__ void read_frags(u32x4 (&F)[12], const Pipe& p, const char* A, const char* B, int hh) {
  const char* a = A + p.a_off + p.frag_off[hh];
  const char* b = B + p.b_off + p.frag_off[hh];
#pragma unroll
  for (int i = 0; i < kBI; ++i) F[i] = *reinterpret_cast<const u32x4*>(a + i * 16 * kRowB);
#pragma unroll
  for (int j = 0; j < kBJ; ++j) F[kBI + j] = *reinterpret_cast<const u32x4*>(b + j * 16 * kRowB);
}

__device__ __forceinline__ void half_mma(TileAcc& acc, const u32x4 (&F)[12]) {
#pragma unroll
  for (int i = 0; i < kBI; ++i)
#pragma unroll
    for (int j = 0; j < kBJ; ++j) acc[i][j] = mfma16x16x32(F[i], F[kBI + j], acc[i][j]);
}

// A phase boundary: nothing is scheduled across it, then the workgroup barrier.
__device__ __forceinline__ void phase_end() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
template <int N>
__device__ __forceinline__ void wait_copies() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_frags() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Copy batch J: the operand with two ring slots for stage J + 1, then the one with three for
// stage J + 2 (stages past the last repeat the last).
__device__ __forceinline__ void copy_batch(const Pipe& p, char* lds, int J, int S) {
  const int t1 = J + 1 < S ? J + 1 : S - 1, t2 = J + 2 < S ? J + 2 : S - 1;
  if constexpr (kARing == 2) {
    copy_op(p.a_src, lds + ((J + 1) % kARing) * kOpB, p.wv_u, t1);
    copy_op(p.b_src, lds + kBOff + ((J + 2) % kBRing) * kOpB, p.wv_u, t2);
  } else {
    copy_op(p.b_src, lds + kBOff + ((J + 1) % kBRing) * kOpB, p.wv_u, t1);
    copy_op(p.a_src, lds + ((J + 2) % kARing) * kOpB, p.wv_u, t2);
  }
}

// The K loop of group G over S stages of 64 features (halves h = 0 .. 2 S - 1 of 32).
//   group 0: phase 2 h multiplies half h, phase 2 h + 1 reads the fragments of half h + 1;
//   group 1: phase 2 h reads the fragments of half h, phase 2 h + 1 multiplies it.
// Copy batch J (tokens of stage J + 1 into token slot (J + 1) % 2, wkv of stage J + 2 into wkv
// slot (J + 2) % 3) is issued by every wave in phase 4 J - 1: both slots held stage J - 1,
// whose last fragments were read in phase 4 J - 2.  At the end of phase 4 J + 2 every wave
// waits until only its wkv copies of batch J are in flight, so the tokens of stage J + 1 and
// the wkv rows of stage J + 1 (batch J - 1) have landed before their first reader (group 0,
// phase 4 J + 3).  Copies past the last stage repeat the last stage into a free slot, so the
// wait counts hold in every phase.
template <int G>
__device__ __forceinline__ void k_loop(TileAcc& acc, const Pipe& p, char* lds, int S) {
  u32x4 F[12];
  // prologue (phase -1): stage 0, wkv stage 1, batch 0; stage 0 lands
  copy_op(p.a_src, lds, p.wv_u, 0);
  copy_op(p.b_src, lds + kBOff, p.wv_u, 0);
  if constexpr (kARing == 3)
    copy_op(p.a_src, lds + kOpB, p.wv_u, S > 1 ? 1 : 0);
  else
    copy_op(p.b_src, lds + kBOff + kOpB, p.wv_u, S > 1 ? 1 : 0);
  copy_batch(p, lds, 0, S);
  wait_copies<3 * kCopies>();
  phase_end();
  if constexpr (G == 0) {
    read_frags(F, p, lds, lds + kBOff, 0);
    wait_frags();
  }
  phase_end();
  int sa = 0, sb = 0;  // ring slots of stage J
  for (int J = 0; J < S; ++J) {
    const char* A = lds + sa * kOpB;
    const char* B = lds + kBOff + sb * kOpB;
    const int na = sa + 1 == kARing ? 0 : sa + 1, nb = sb + 1 == kBRing ? 0 : sb + 1;  // stage J + 1
    if constexpr (G == 0) {
      half_mma(acc, F);                                           // 4 J: half 2 J
      phase_end();
      read_frags(F, p, A, B, 1);                                  // 4 J + 1: read half 2 J + 1
      wait_frags();
      phase_end();
      half_mma(acc, F);                                           // 4 J + 2: half 2 J + 1
      wait_copies<kCopies>();
      phase_end();
      copy_batch(p, lds, J + 1, S);                               // 4 J + 3: read half 2 J + 2
      read_frags(F, p, lds + na * kOpB, lds + kBOff + nb * kOpB, 0);
      wait_frags();
      phase_end();
    } else {
      read_frags(F, p, A, B, 0);                                  // 4 J: read half 2 J
      wait_frags();
      phase_end();
      half_mma(acc, F);                                           // 4 J + 1: half 2 J
      phase_end();
      read_frags(F, p, A, B, 1);                                  // 4 J + 2: read half 2 J + 1
      wait_frags();
      wait_copies<kCopies>();
      phase_end();
      copy_batch(p, lds, J + 1, S);                               // 4 J + 3: half 2 J + 1
      half_mma(acc, F);
      phase_end();
    }
    sa = na;
    sb = nb;
  }
  // the repeated copies may still be landing: every copy done before LDS is reused
  wait_copies<0>();
  phase_end();
}

// Stages [s0, s0 + ns) of the tile's K loop.
__device__ __forceinline__ void tile_gemm(TileAcc& acc, const TiledArgs& a, char* lds, int64_t m0, int n0, int s0,
                                          int ns, int tid) {
  const int lane = tid & 63, wv = tid >> 6;
  Pipe p;
  p.wv_u = __builtin_amdgcn_readfirstlane(wv);
  {
    const int rr = lane >> 3, chunk = (lane & 7) ^ rr;
    const size_t row_bytes = size_t(a.K) * 2;
    const size_t k0 = size_t(s0) * kRowB;
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int r = (4 * p.wv_u + i) * 8 + rr;  // row of the tile
      p.a_src[i] = reinterpret_cast<const char*>(a.wkv) + size_t(n0 + r) * row_bytes + k0 + 16 * chunk;
      int64_t m = m0 + r;
      m = m < a.M ? m : a.M - 1;  // rows past the last token repeat it (their results are dropped)
      p.b_src[i] = reinterpret_cast<const char*>(a.emb) + size_t(m) * row_bytes + k0 + 16 * chunk;
    }
  }
  {
    const int r = lane & 15;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) p.frag_off[hh] = uint32_t(r * kRowB + 16 * ((4 * hh + (lane >> 4)) ^ (r & 7)));
  }
  p.a_off = (wv >> 2) * 128 * kRowB;
  p.b_off = (wv & 3) * 64 * kRowB;
#pragma unroll
  for (int i = 0; i < kBI; ++i)
#pragma unroll
    for (int j = 0; j < kBJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (__builtin_amdgcn_readfirstlane(wv) < 4)
    k_loop<0>(acc, p, lds, ns);
  else
    k_loop<1>(acc, p, lds, ns);
}

// ---------------------------------------------------------------- fp8 schedule
constexpr int kMxK = 128;                        // features per stage
constexpr int kMxScaleOff = 4 * kOpB;            // scale slots: wkv 2 x 1 KB, then tokens 2 x 1 KB
constexpr int kMxBOff = 2 * kOpB;                // token ring offset
static_assert(kMxScaleOff + 4096 <= kLds, "fp8 schedule LDS");

struct PipeMx {
  const char* a_src[kCopies];  // per-lane global source of each wkv copy at stage 0
  const char* b_src[kCopies];  // the same for the token copies
  const char* s_src;           // this lane's scale dword source at stage 0 (wkv rows for waves 0-3)
  uint32_t s_dst;              // byte offset of the wave's 256 scale bytes within a scale slot pair
  uint32_t lo_off, hi_off;     // per-lane offsets of the two 16-byte parts of a fragment read
  int wv_u;
  int a_off, b_off;            // byte offsets of this wave's first wkv row and first token row
  int sa_off, sb_off;          // byte offsets of their scale dwords in a scale slot
};

// Copies of one stage of the fp8 schedule, each wave its share, into ring slot `slot`; `t` is the
// stage copied (past the last stage the last one is repeated into the free slot, so that every
// phase issues the same number of copies).  Tokens: rows 32 w .. 32 w + 31 (4 instructions);
// wkv: the same rows, so waves 0-3 copy the rows of group 0 and waves 4-7 those of group 1
// (4 instructions); scales: one instruction, waves 0-3 the wkv rows' dwords, 4-7 the tokens'.
__device__ __forceinline__ void copy_b_mx(const PipeMx& p, char* lds, int t, int slot) {
  copy_op(p.b_src, lds + kMxBOff + slot * kOpB, p.wv_u, t);
}
__device__ __forceinline__ void copy_a_mx(const PipeMx& p, char* lds, int t, int slot) {
  copy_op(p.a_src, lds + slot * kOpB, p.wv_u, t);
}
__device__ __forceinline__ void copy_s_mx(const PipeMx& p, char* lds, int t, int slot) {
  __builtin_amdgcn_global_load_lds((const void*)(p.s_src + size_t(t) * 4),
                                   (lds_ptr_t)(lds + kMxScaleOff + slot * 1024 + p.s_dst), 4, 0, 0);
}

struct FragMx {
  i32x8 a[4];  // wkv row blocks of the half stage: parts l / 16, l / 16 + 4
  int sa[4];
  i32x8 b[4];  // token blocks
  int sb[4];
};

__device__ __forceinline__ int scale_byte(uint32_t dw, int lane) { return int((dw >> (8 * (lane >> 4))) & 0xFFu); }

// wkv fragments of half hh (row blocks 4 hh .. 4 hh + 3 of the wave's 8) of the stage in slot r.
__device__ __forceinline__ void read_a_mx(FragMx& F, const PipeMx& p, const char* lds, int r, int hh, int lane) {
  const char* A = lds + r * kOpB + p.a_off;
  const char* S = lds + kMxScaleOff + r * 1024 + p.sa_off;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * hh + k;
    F.a[k] = mx_operand(*reinterpret_cast<const u32x4*>(A + i * 16 * kRowB + p.lo_off),
                        *reinterpret_cast<const u32x4*>(A + i * 16 * kRowB + p.hi_off));
    F.sa[k] = scale_byte(*reinterpret_cast<const uint32_t*>(S + i * 64), lane);
  }
}
__device__ __forceinline__ void read_b_mx(FragMx& F, const PipeMx& p, const char* lds, int r, int lane) {
  const char* B = lds + kMxBOff + r * kOpB + p.b_off;
  const char* S = lds + kMxScaleOff + 2048 + r * 1024 + p.sb_off;
#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    F.b[j] = mx_operand(*reinterpret_cast<const u32x4*>(B + j * 16 * kRowB + p.lo_off),
                        *reinterpret_cast<const u32x4*>(B + j * 16 * kRowB + p.hi_off));
    F.sb[j] = scale_byte(*reinterpret_cast<const uint32_t*>(S + j * 64), lane);
  }
}
// (The empty asm statements pin the MFMAs to their phase: otherwise the compiler sinks them
// past the phase barrier, next to the following phase's fragment reads, with both halves'
// fragments live at once.)
__device__ __forceinline__ void half_mma_mx(TileAcc& acc, const FragMx& F, int hh) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < kBJ; ++j)
      acc[4 * hh + k][j] = mfma_mx16x16x128(F.a[k], F.sa[k], F.b[j], F.sb[j], acc[4 * hh + k][j]);
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < kBJ; ++j) asm volatile("" : "+v"(acc[4 * hh + k][j]));
}

// The fp8 K loop of group G over S stages of 128 features, rings of two slots:
//   group 0: phase 4 J multiplies half 0 of stage J, 4 J + 1 reads half 1, 4 J + 2 multiplies
//            it, 4 J + 3 reads half 0 (and the token fragments and scales) of stage J + 1;
//   group 1: phase 4 J reads half 0 (and the token fragments and scales) of stage J, 4 J + 1
//            multiplies it, 4 J + 2 reads half 1, 4 J + 3 multiplies it.
// Each part of stage J + 2 is copied into stage J's slot as soon as stage J's last reader of that
// part is done: the tokens and their scales are read once per stage (last in phase 4 J), so they
// are copied in phase 4 J + 1; the wkv rows of group 0 in phase 4 J + 2, those of group 1 and the
// wkv scales in phase 4 J + 3.  Stage J + 2 is first read in phase 4 J + 7.  At the end of phase
// 4 J + 2 each wave waits until only its copies of stage J + 2 are in flight (group 0: tokens and
// wkv rows, 8 instructions; group 1: tokens and their scales, 5), so stage J + 1 has landed
// everywhere before group 0 reads it in phase 4 J + 3.
template <int G>
__device__ __forceinline__ void k_loop_mx(TileAcc& acc, const PipeMx& p, char* lds, int S, int lane) {
  FragMx F;
  // prologue: stages 0 and 1 (9 copies each); stage 0 lands
  for (int t = 0; t < 2; ++t) {
    const int ts = t < S ? t : S - 1;
    copy_b_mx(p, lds, ts, t);
    copy_a_mx(p, lds, ts, t);
    copy_s_mx(p, lds, ts, t);
  }
  wait_copies<9>();
  phase_end();
  if constexpr (G == 0) {
    read_a_mx(F, p, lds, 0, 0, lane);
    read_b_mx(F, p, lds, 0, lane);
    wait_frags();
  }
  phase_end();
  for (int J = 0; J < S; ++J) {
    const int r = J & 1;
    const int t2 = J + 2 < S ? J + 2 : S - 1;  // the stage copied into slot r
    if constexpr (G == 0) {
      half_mma_mx(acc, F, 0);                                     // 4 J
      phase_end();
      copy_b_mx(p, lds, t2, r);                                   // 4 J + 1
      read_a_mx(F, p, lds, r, 1, lane);
      wait_frags();
      phase_end();
      copy_a_mx(p, lds, t2, r);                                   // 4 J + 2
      half_mma_mx(acc, F, 1);
      wait_copies<8>();
      phase_end();
      copy_s_mx(p, lds, t2, r);                                   // 4 J + 3
      if (J + 1 < S) {
        read_a_mx(F, p, lds, r ^ 1, 0, lane);
        read_b_mx(F, p, lds, r ^ 1, lane);
        wait_frags();
      }
      phase_end();
    } else {
      read_a_mx(F, p, lds, r, 0, lane);                           // 4 J
      read_b_mx(F, p, lds, r, lane);
      wait_frags();
      phase_end();
      copy_b_mx(p, lds, t2, r);                                   // 4 J + 1
      copy_s_mx(p, lds, t2, r);
      half_mma_mx(acc, F, 0);
      phase_end();
      read_a_mx(F, p, lds, r, 1, lane);                           // 4 J + 2
      wait_frags();
      wait_copies<5>();
      phase_end();
      copy_a_mx(p, lds, t2, r);                                   // 4 J + 3
      half_mma_mx(acc, F, 1);
      phase_end();
    }
  }
  // the repeated copies may still be landing: every copy done before LDS is reused
  wait_copies<0>();
  phase_end();
}

// Stages [s0, s0 + ns) of the tile's fp8 K loop.
__device__ __forceinline__ void tile_gemm_mx(TileAcc& acc, const TiledArgs& a, char* lds, int64_t m0, int n0, int s0,
                                             int ns, int tid) {
  const int lane = tid & 63, wv = tid >> 6;
  PipeMx p;
  p.wv_u = __builtin_amdgcn_readfirstlane(wv);
  const size_t k0 = size_t(s0) * kMxK;
  {
    const int rr = lane >> 3, chunk = (lane & 7) ^ rr;
    const size_t row_bytes = size_t(a.K);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int r = (4 * p.wv_u + i) * 8 + rr;  // row of the tile
      p.a_src[i] = reinterpret_cast<const char*>(a.wkv8) + size_t(n0 + r) * row_bytes + k0 + 16 * chunk;
      int64_t m = m0 + r;
      m = m < a.M ? m : a.M - 1;  // rows past the last token repeat it (their results are dropped)
      p.b_src[i] = reinterpret_cast<const char*>(a.tok8) + size_t(m) * row_bytes + k0 + 16 * chunk;
    }
  }
  {
    // scale dwords: waves 0-3 the wkv rows 64 (w & 3) + l, waves 4-7 the token rows
    const size_t srow = size_t(a.K / 32);
    const int r = 64 * (p.wv_u & 3) + lane;
    if (p.wv_u < 4) {
      p.s_src = reinterpret_cast<const char*>(a.wkv8s) + size_t(n0 + r) * srow + k0 / 32;
      p.s_dst = uint32_t(256 * (p.wv_u & 3));
    } else {
      int64_t m = m0 + r;
      m = m < a.M ? m : a.M - 1;
      p.s_src = reinterpret_cast<const char*>(a.tok8s) + size_t(m) * srow + k0 / 32;
      p.s_dst = uint32_t(2048 + 256 * (p.wv_u & 3));
    }
  }
  {
    const int r = lane & 15, g = lane >> 4;
    p.lo_off = uint32_t(r * kRowB + 16 * (g ^ (r & 7)));
    p.hi_off = uint32_t(r * kRowB + 16 * ((g + 4) ^ (r & 7)));
    p.a_off = (wv >> 2) * 128 * kRowB;
    p.b_off = (wv & 3) * 64 * kRowB;
    p.sa_off = ((wv >> 2) * 128 + r) * 4;
    p.sb_off = ((wv & 3) * 64 + r) * 4;
  }
#pragma unroll
  for (int i = 0; i < kBI; ++i)
#pragma unroll
    for (int j = 0; j < kBJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (__builtin_amdgcn_readfirstlane(wv) < 4)
    k_loop_mx<0>(acc, p, lds, ns, lane);
  else
    k_loop_mx<1>(acc, p, lds, ns, lane);
}

// ---------------------------------------------------------------- split K
// Tile t's two workgroups share two control words at split_off + 64 t: arrivals and "partial
// written".  The first to arrive stores its fp32 partial tile (16-byte device-coherent stores,
// one 1 KB run per wave instruction), waits for the stores to complete, sets the second word and
// exits; the second waits for that word (its partner has already arrived and never waits), adds
// the partial to its own accumulators, clears both words and finishes the tile.  The sum of two
// fp32 values does not depend on their order, so the result does not depend on which half
// arrives first.  (The partial's offsets are a per-lane part and a scalar part per block.)
// Returns false in the workgroup that exits.
__device__ __forceinline__ bool split_merge(TileAcc& acc, const TiledArgs& a, int64_t tile, char* lds, int tid) {
  uint32_t* w = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(a.ws) + a.split_off + size_t(tile) * 64);
  int* flag = reinterpret_cast<int*>(lds + kLds - 4);  // past every LDS user of the epilogue
  if (tid == 0) *flag = int(atomic_add_relaxed(w, 1u));
  __syncthreads();
  const bool first = *flag == 0;
  const __amdgpu_buffer_rsrc_t pr = coherent_rsrc(a.kpart + size_t(tile) * (kTM * kTN));
  if (first) {
#pragma unroll
    for (int i = 0; i < kBI; ++i)
#pragma unroll
      for (int j = 0; j < kBJ; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), pr, uint32_t(tid * 16),
                                               (i * kBJ + j) * kThreads * 16, kCpolSc1);
    drain_memory_ops();
    __syncthreads();
    if (tid == 0) store_relaxed(w + 1, 1u);
    return false;
  }
  if (tid == 0) {
    uint32_t it = 0;
    while (load_relaxed(w + 1) == 0u) {
      __builtin_amdgcn_s_sleep(2);
      if (++it > a.spin_budget) {
        atomic_add_relaxed(reinterpret_cast<uint32_t*>(a.ws), 1u);
        break;
      }
    }
    store_relaxed(w, 0u);
    store_relaxed(w + 1, 0u);
  }
  __syncthreads();
  // one row block (4 loads) at a time: the accumulators already fill most of the registers
#pragma unroll
  for (int i = 0; i < kBI; ++i) {
#pragma unroll
    for (int j = 0; j < kBJ; ++j)
      acc[i][j] += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, uint32_t(tid * 16),
                                                                                (i * kBJ + j) * kThreads * 16,
                                                                                kCpolSc1));
    asm volatile("" ::: "memory");
  }
  __syncthreads();  // the flag word is reused by the epilogue's LDS
  return true;
}

// ---------------------------------------------------------------- epilogues
// After the K loop the accumulator tile goes to LDS as bf16 (the rounding the projection output
// has): 256 token rows of 512 bytes, 16-byte chunk c of row t at position c ^ (t & 31).  The
// epilogues then walk token rows with half a wave per row (32 lanes x 8 features), so every
// global access of x, out and kv is 16 bytes per lane and 512 contiguous bytes per row.
constexpr int kVRow = kTN * 2;                     // bytes per token row
constexpr int kVBytes = kTM * kVRow;               // 128 KB
constexpr int kGateOff = kVBytes;                  // value tiles: gates [4][256] fp32
constexpr int kFlagOff = kGateOff + 4 * kTM * 4;   // key tiles: last-arriver flag
static_assert(kFlagOff + 4 <= kLds, "epilogue LDS");

__device__ __forceinline__ int vswz(int t, int c) { return t * kVRow + 16 * (c ^ (t & 31)); }

// Accumulator block (i, j) of wave (wr, wt) holds columns 128 wr + 16 i + 4 (l >> 4) + 0..3 of
// token 64 wt + 16 j + (l & 15).
__device__ __forceinline__ void acc_to_lds(const TileAcc& acc, char* V, int lane, int wr, int wt) {
#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    const int t = 64 * wt + 16 * j + (lane & 15);
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
      const int f = 128 * wr + 16 * i + 4 * (lane >> 4);
      *reinterpret_cast<u32x2*>(V + vswz(t, f >> 3) + 2 * (f & 7)) =
          u32x2{pack_bf16x2(acc[i][j].x, acc[i][j].y), pack_bf16x2(acc[i][j].z, acc[i][j].w)};
    }
  }
}

__device__ __forceinline__ void unpack8(u32x4 w, float (&v)[8]) {
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

// Projection alone: the tile's kv rows, 512 contiguous bytes per token.
__device__ __forceinline__ void kv_epilogue(const TiledArgs& a, const char* V, int64_t m0, int n0, int tid) {
  const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, half = lane >> 5;
#pragma unroll 4
  for (int p = 0; p < 16; ++p) {
    const int t = p * 16 + wv * 2 + half;
    const int64_t m = m0 + t;
    if (m < a.M)
      *reinterpret_cast<u32x4*>(a.kv + m * a.N + n0 + 8 * l32) = *reinterpret_cast<const u32x4*>(V + vswz(t, l32));
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

// Key tile (stream s, features dseg .. dseg + 255 of the stream): per token, this tile's share
// of the gate's three sums (|h|^2, |key|^2 and sum h * q * k * key) is posted to the workspace;
// the last of the stream's key tiles sums the shares in column-block order, evaluates the 256
// gates and hands them to the value tiles of the token block.
__device__ __forceinline__ void key_epilogue(const TiledArgs& a, char* lds, int64_t tb, int64_t m0, int s, int cbs,
                                             int dseg, int tid) {
  const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const char* V = lds;
  int* flag = reinterpret_cast<int*>(lds + kFlagOff);
  const int d = dseg + 8 * l32;
  float wq[8];
  {
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(a.q_weight + s * a.dim + d);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(a.q_weight + s * a.dim + d + 4);
    const f32x4 k0 = *reinterpret_cast<const f32x4*>(a.k_weight + s * a.dim + d);
    const f32x4 k1 = *reinterpret_cast<const f32x4*>(a.k_weight + s * a.dim + d + 4);
    wq[0] = q0.x * k0.x; wq[1] = q0.y * k0.y; wq[2] = q0.z * k0.z; wq[3] = q0.w * k0.w;
    wq[4] = q1.x * k1.x; wq[5] = q1.y * k1.y; wq[6] = q1.z * k1.z; wq[7] = q1.w * k1.w;
  }
  float* P = tpartial(a, tb, s, cbs);
  // 16 passes of 16 rows (8 waves x 2 half-waves); the x loads of all 16 are in flight at once
  // (the accumulators are in LDS by now, so the registers are free: one memory round trip)
#pragma unroll
  for (int p0 = 0; p0 < 16; p0 += 16) {
    u32x4 xv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int t = (p0 + q) * 16 + wv * 2 + half;
      const int64_t m = m0 + t;
      const int64_t mm = m < a.M ? m : a.M - 1;
      xv[q] = *reinterpret_cast<const u32x4*>(a.x + (mm * 4 + s) * a.dim + d);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int t = (p0 + q) * 16 + wv * 2 + half;
      float h[8], key[8];
      unpack8(xv[q], h);
      unpack8(*reinterpret_cast<const u32x4*>(V + vswz(t, l32)), key);
      float sa = 0.f, sk = 0.f, sd = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sa += h[e] * h[e];
        sk += key[e] * key[e];
        sd += (h[e] * wq[e]) * key[e];
      }
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        sa += __shfl_xor(sa, o, 64);
        sk += __shfl_xor(sk, o, 64);
        sd += __shfl_xor(sd, o, 64);
      }
      if (l32 == 0) {
        store_coherent(P + t * 3 + 0, sa);
        store_coherent(P + t * 3 + 1, sk);
        store_coherent(P + t * 3 + 2, sd);
      }
    }
  }
  drain_memory_ops();
  __syncthreads();
  if (tid == 0) *flag = (atomic_add_relaxed(tcounter(a, tb, s), 1u) == uint32_t(a.n_vcb - 1)) ? 1 : 0;
  __syncthreads();
  if (*flag && tid < kTM) {
    // every column block of this stream has posted: sum in column-block order
    float A = 0.f, Kq = 0.f, D = 0.f;
    for (int base = 0; base < a.n_vcb; base += 8) {
      float v[8][3];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int c = base + q < a.n_vcb ? base + q : base;
        const float* Pc = tpartial(a, tb, s, c) + tid * 3;
        v[q][0] = load_coherent(Pc + 0);
        v[q][1] = load_coherent(Pc + 1);
        v[q][2] = load_coherent(Pc + 2);
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
    // the partials are consumed: leave them zero, so that the control words are all zero again
    // after the call (any schedule may use them next)
    for (int c = 0; c < a.n_vcb; ++c) {
      float* Pc = tpartial(a, tb, s, c) + tid * 3;
      store_coherent(Pc + 0, 0.0f);
      store_coherent(Pc + 1, 0.0f);
      store_coherent(Pc + 2, 0.0f);
    }
  }
}

// Value tile (features dseg .. dseg + 255 of the value): wait for the 4 x 256 gates of the
// token block, then out = h + gate * value on every stream.
__device__ __forceinline__ void value_epilogue(const TiledArgs& a, char* lds, int64_t tb, int64_t m0, int cbs,
                                               int dseg, int tid) {
  const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const char* V = lds;
  float (*gates)[kTM] = reinterpret_cast<float (*)[kTM]>(lds + kGateOff);
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
  const int d = dseg + 8 * l32;
  // 1024 rows (token r >> 2, stream r & 3) in 64 passes of 16; 32 passes of x loads in flight
  // (two memory round trips per tile)
  for (int p0 = 0; p0 < 64; p0 += 32) {
    u32x4 xv[32];
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      const int r = (p0 + q) * 16 + wv * 2 + half;
      const int64_t m = m0 + (r >> 2);
      const int64_t mm = m < a.M ? m : a.M - 1;
      xv[q] = *reinterpret_cast<const u32x4*>(a.x + (mm * 4 + (r & 3)) * a.dim + d);
    }
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      const int r = (p0 + q) * 16 + wv * 2 + half;
      const int t = r >> 2, s2 = r & 3;
      const int64_t m = m0 + t;
      if (m >= a.M) continue;
      const bool open = a.token_mask == nullptr || a.token_mask[m] != 0;
      uint16_t* dst = a.out + (m * 4 + s2) * a.dim + d;
      if (!open) {
        if (a.out != a.x) *reinterpret_cast<u32x4*>(dst) = xv[q];
        continue;
      }
      float h[8], v[8];
      unpack8(xv[q], h);
      unpack8(*reinterpret_cast<const u32x4*>(V + vswz(t, l32)), v);
      const float g = gates[s2][t];
      *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16x2(h[0] + g * v[0], h[1] + g * v[1]),
                                             pack_bf16x2(h[2] + g * v[2], h[3] + g * v[3]),
                                             pack_bf16x2(h[4] + g * v[4], h[5] + g * v[5]),
                                             pack_bf16x2(h[6] + g * v[6], h[7] + g * v[7])};
    }
  }
}

template <bool FUSED, bool MX = false>
__global__ __launch_bounds__(kThreads) void k_tiled(TiledArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t n_tb = (a.M + kTM - 1) / kTM;
  // the tile: workgroups from split_from on take half of K of a split tile.  They come in runs
  // of 16 (the last run shorter): half 0 of 8 consecutive split tiles, then half 1 of the same 8,
  // so that both halves of tile b run on the XCD that the tile order gives b (workgroup ids are
  // dealt to the 8 XCDs round robin)
  const int64_t bi = int64_t(blockIdx.x);
  const bool split = FUSED && bi >= a.split_from;
  int64_t b = bi;
  int half_k = -1;
  if (split) {
    const int64_t rel = bi - a.split_from, q = rel >> 4, n_wg = int64_t(gridDim.x) - a.split_from;
    const int64_t run = n_wg - 16 * q >= 16 ? 8 : (n_wg - 16 * q) >> 1;  // tiles in this run
    const int64_t w = rel - 16 * q;
    half_k = int(w / run);
    b = a.split_from + 8 * q + (w - half_k * run);
  }
  const int64_t per_group = int64_t(kGroupTb) * (a.N / kTN);
  const int64_t g = b / per_group;
  const int64_t g_size = n_tb - g * kGroupTb < kGroupTb ? n_tb - g * kGroupTb : kGroupTb;
  const int64_t local = b - g * per_group;
  const int64_t tb = g * kGroupTb + local % g_size;
  const int cb = int(local / g_size);
  const int64_t m0 = tb * kTM;
  const int n0 = cb * kTN;

  TileAcc acc;
  const int S = a.K / (MX ? kMxK : kTK), sh = S / 2;
  const int s0 = half_k <= 0 ? 0 : sh;
  const int ns = half_k < 0 ? S : (half_k == 0 ? sh : S - sh);
  if constexpr (MX) tile_gemm_mx(acc, a, lds, m0, n0, s0, ns, tid);
  else tile_gemm(acc, a, lds, m0, n0, s0, ns, tid);
  if (half_k >= 0 && !split_merge(acc, a, b - a.split_from, lds, tid)) return;
  // the K loop ended with a barrier after its last LDS access: the ring is free
  acc_to_lds(acc, lds, lane, wv >> 2, wv & 3);
  __syncthreads();
  if constexpr (!FUSED) {
    kv_epilogue(a, lds, m0, n0, tid);
  } else {
    const int s = n0 / a.dim;  // a tile lies in one segment: dim is a multiple of 256
    const int dseg = n0 - s * a.dim;
    const int cbs = dseg / kTN;
    if (s < 4)
      key_epilogue(a, lds, tb, m0, s, cbs, dseg, tid);
    else
      value_epilogue(a, lds, tb, m0, cbs, dseg, tid);
  }
}

hipError_t launch_tiled_impl(const TiledArgs& a, bool fused, hipStream_t stream) {
  const int64_t n_tb = (a.M + kTM - 1) / kTM;
  int64_t tiles = n_tb * (a.N / kTN);
  if (fused) {
    if (a.split_from < 0 || a.split_from > tiles || tiles - a.split_from > kSplitMaxTiles) return hipErrorInvalidValue;
    tiles += tiles - a.split_from;  // one more workgroup per split tile
  }
  if (tiles <= 0 || tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.mx && !fused) return hipErrorInvalidValue;
  const void* fn = a.mx ? reinterpret_cast<const void*>(&k_tiled<true, true>)
                        : fused ? reinterpret_cast<const void*>(&k_tiled<true>)
                                : reinterpret_cast<const void*>(&k_tiled<false>);
  const int kind = a.mx ? 2 : (fused ? 1 : 0);
  static bool attr_set[3] = {false, false, false};
  if (!attr_set[kind]) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    attr_set[kind] = true;
  }
  TiledArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(fn, dim3(unsigned(tiles)), dim3(kThreads), params, kLds, stream);
}

// The first split tile: every tile while they fill at most half of a 256-CU device; else, in
// the bf16 schedule, the tiles of the last, partial round when they fill at most half of the
// device (so that their halves fit in one round); tiles (no split) otherwise.  (Measured at 8192
// tokens in same-process A/Bs: the bf16 forward 2243 -> 2200 us with its last 128 tiles split;
// the fp8 forward 1391 -> 1432 us, so the fp8 schedule does not split a last round.)
int64_t tiled_split_from(int64_t M, int N, int K, bool mx, int cus) {
  const int64_t tiles = (M + kTM - 1) / kTM * (N / kTN);
  if (K / (mx ? kMxK : kTK) < 2) return tiles;
  if (tiles <= kSplitMaxTiles) return 0;
  const int64_t r = cus > 0 ? tiles % cus : 0;
  return !mx && r > 0 && r <= kSplitMaxTiles && 2 * r <= cus ? tiles - r : tiles;
}

// Control words of the fused schedule: header, per-(token block, stream) counters, split-K
// words (a fixed 64 bytes for each of up to kSplitMaxTiles tiles), gate slots, partial sums.
// All zero before and after every call.
size_t tiled_control_layout(TiledArgs* a, int64_t M, int dim) {
  const int64_t n_tb = (M + kTM - 1) / kTM;
  const int n_vcb = dim / kTN;
  size_t off = 256 + size_t(n_tb) * 4 * 256;  // header, counters (one 256-byte line each)
  const size_t split_off = off;
  off += size_t(kSplitMaxTiles) * 64;
  const size_t slot_off = off;
  off += size_t(n_tb) * n_vcb * 4 * kTM * 4;
  off = (off + 255) & ~size_t(255);
  const size_t part_off = off;
  off += size_t(n_tb) * 4 * n_vcb * kTM * 3 * 4;
  if (a != nullptr) {
    a->n_vcb = n_vcb;
    a->split_off = split_off;
    a->slot_off = slot_off;
    a->part_off = part_off;
  }
  return off;
}

// fp32 partial tiles of split K: room for the most tiles any call splits (a fixed amount per
// layout, so the staging size does not decrease with M).
size_t split_partial_bytes(int N) {
  if (N / kTN <= 0) return 0;
  return size_t(kSplitMaxTiles) * kTM * kTN * 4;
}

}  // namespace

bool tiled_shape_ok(int N, int K, int dim, bool fused) {  // K: stages of 64 features
  if (N % kTN != 0 || K % kTK != 0) return false;
  if (fused && dim % kTN != 0) return false;
  return true;
}

bool tiled_mx_ok(int N, int K, int dim, int scale_block) {
  return tiled_shape_ok(N, K, dim, true) && K % kMxK == 0 && scale_block % 32 == 0;
}

size_t tiled_control_bytes(int64_t M, int dim) { return tiled_control_layout(nullptr, M, dim); }

size_t tiled_staging_bytes(int64_t M, int K, int N) {
  return ((size_t(M) * K * 2 + 255) & ~size_t(255)) + split_partial_bytes(N);
}

// fp8 schedule: codes [M, K], then E8M0 scales [M, K / 32], then the split partial tiles
size_t mx_codes_bytes(int64_t M, int K) { return (size_t(M) * K + 255) & ~size_t(255); }
size_t mx_scales_bytes(int64_t M, int K) { return (size_t(M) * (K / 32) + 255) & ~size_t(255); }
size_t tiled_staging_bytes_mx(int64_t M, int K, int N) {
  return mx_codes_bytes(M, K) + mx_scales_bytes(M, K) + split_partial_bytes(N);
}

hipError_t launch_kv_proj_tiled(const TiledArgs& a, hipStream_t stream) { return launch_tiled_impl(a, false, stream); }

hipError_t launch_forward_tiled(TiledArgs a, const GatherArgs& g, void* workspace, void* staging, int num_cus,
                                hipStream_t stream) {
  GatherArgs ga = g;
  char* stg = static_cast<char*>(staging);
  hipError_t e;
  if (a.mx) {
    uint8_t* codes8 = reinterpret_cast<uint8_t*>(stg);
    uint8_t* scales8 = reinterpret_cast<uint8_t*>(stg + mx_codes_bytes(a.M, a.K));
    e = launch_gather_mx(ga, codes8, scales8, stream);
    a.tok8 = codes8;
    a.tok8s = scales8;
    a.kpart = reinterpret_cast<float*>(stg + mx_codes_bytes(a.M, a.K) + mx_scales_bytes(a.M, a.K));
  } else {
    ga.emb = reinterpret_cast<uint16_t*>(staging);
    e = launch_gather_dequant(ga, stream);
    a.emb = reinterpret_cast<const uint16_t*>(staging);
    a.kpart = reinterpret_cast<float*>(stg + ((size_t(a.M) * a.K * 2 + 255) & ~size_t(255)));
  }
  if (e != hipSuccess) return e;
  a.ws = workspace;
  tiled_control_layout(&a, a.M, a.dim);
  a.split_from = tiled_split_from(a.M, a.N, a.K, a.mx != 0, num_cus);
  return launch_tiled_impl(a, true, stream);
}

}  // namespace engram
