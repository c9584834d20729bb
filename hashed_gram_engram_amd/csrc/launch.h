// Kernel argument blocks and launchers (host side of the HIP kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace engram {

struct GatherArgs {
  const uint8_t* table;
  const void* scales;  // fp32, or E8M0 bytes when scale_e8m0
  const int64_t* hash_ids;
  int64_t n_pairs;  // tokens * n_cols
  int head_dim;
  int scale_block;
  int scale_e8m0;
  int64_t n_rows;
  uint16_t* emb;
  int32_t* err_count;
  // frag_cols > 0: emb in the 16 x 16 x 32 MFMA operand order of a table of frag_cols columns
  // (1 KB per 16 tokens x 32 features: lane l's 16 bytes, token l % 16, features 8 (l / 16) ..),
  // and the rows of the pairs n_pairs .. n_fill - 1 written as zeros
  int frag_cols;
  int64_t n_fill;
};

struct GateArgs {
  const uint16_t* x;
  const uint16_t* kv;
  const float* q_weight;
  const float* k_weight;
  const uint8_t* token_mask;
  int64_t M;
  int dim;
  float eps, clamp, inv_sqrt_dim;
  uint16_t* out;
  float* gate;
};

// Arguments of the weight-streaming projection kernels (projection alone, or the whole
// Engram forward).  Token blocks are 64 tokens; the grid is persistent.
struct StreamArgs {
  const uint16_t* wkv;  // [N, K] bf16
  // or, when w8, MXFP8 weights: e4m3fn codes [N, K] and E8M0 scales [N, K / 32]
  const uint8_t* wkv8;
  const uint8_t* wkv8s;
  int w8;
  int64_t M;
  int K, N, dim;
  // projection alone
  const uint16_t* emb;  // [M, K] bf16
  uint16_t* kv;         // [M, N] bf16
  // whole forward
  const uint16_t* x;
  const int64_t* hash_ids;
  const uint8_t* token_mask;
  const uint8_t* table;
  const void* scales;  // fp32, or E8M0 bytes when scale_e8m0
  const float* q_weight;
  const float* k_weight;
  uint16_t* out;
  int32_t* err_count;
  int n_cols, head_dim, scale_block, scale_e8m0;
  int64_t n_rows;
  float eps, clamp, inv_sqrt_dim;
  // workspace views
  uint32_t* ws_hdr;    // workspace start: [0] wait time-outs, then per-token-block blocks
  size_t tb_stride;    // bytes per token-block block
  uint32_t spin_budget;
  // grid: G streaming workgroups, then (fused forward of one or two token blocks) n_apply
  // workgroups that apply the gates to the value rows, n_apply / n_atb of them per token block
  int G, n_apply, n_atb;
};

// The hash step: token ids -> row ids of every Engram layer.
constexpr int64_t kDead = -1;  // compressed id of a token that takes no part in an n-gram
struct HashArgs {
  const uint32_t* token_map;   // [vocab]
  const int64_t* multipliers;  // [n_layers, max_ngram]
  const int64_t* primes;       // [n_layers, max_ngram - 1, n_heads]
  const int64_t* offsets;      // [n_layers, (max_ngram - 1) * n_heads]
  const int64_t* input_ids;    // [B, L]
  const uint8_t* token_mask;   // [B, L] or null
  int64_t* history;            // [B, history_len]
  int64_t* hash_ids;           // [n_layers, B, L, (max_ngram - 1) * n_heads]
  int32_t* err_count;
  int64_t B, L, start_pos, vocab, history_len;
  int n_layers, max_ngram, n_heads, pad_id;
};
hipError_t launch_hash_ids(const HashArgs& a, hipStream_t stream);

hipError_t launch_gather_dequant(const GatherArgs& a, hipStream_t stream);
// Gather without dequantisation (E8M0 tables): codes [pairs, head_dim] to codes8 and one E8M0
// byte per 32 features to scales8 [pairs, head_dim / 32]; rows that read as zeros get zero codes
// and scale 127 (2^0).
hipError_t launch_gather_mx(const GatherArgs& a, uint8_t* codes8, uint8_t* scales8, hipStream_t stream);
hipError_t launch_gate_apply(const GateArgs& a, hipStream_t stream);

// Projection alone: kv = bf16(emb @ wkv^T).
hipError_t launch_kv_proj_stream(const StreamArgs& a, int num_cus, hipStream_t stream);

// Whole forward, weight-streaming schedule.  Needs a zero-filled workspace of
// stream_workspace_bytes() whose control words are zero (the kernel leaves them zero).
size_t stream_workspace_bytes(int64_t M, int N, int dim, int grid);
int stream_grid(int N, int num_cus);
// Most rows of wkv one workgroup of the weight-streaming schedule owns.
int stream_rows_per_group(int N, int G);
hipError_t launch_forward_stream(StreamArgs a, void* workspace, int num_cus, hipStream_t stream);
// 65..128 tokens in one pass over bf16 weights (workspace as the streaming kernel's, two blocks)
bool stream_tb2_ok(int K, int N, int dim, int n_cols, int head_dim, int scale_block, int num_cus);
hipError_t launch_forward_tb2(StreamArgs a, void* workspace, int num_cus, hipStream_t stream);
// 129..256 tokens in one pass over bf16 weights, from tokens gathered into a.emb beforehand
// (bf16 in the MFMA operand order, GatherArgs::frag_cols; workspace as the streaming kernel's, up
// to four blocks)
bool stream_tb4_ok(int K, int N, int dim, int num_cus);
hipError_t launch_forward_tb4(StreamArgs a, void* workspace, int num_cus, hipStream_t stream);
// Whether the weight-streaming kernels take MXFP8 weights for this shape (the wide K loop:
// K / 4 a multiple of 128, 1..7 row blocks per workgroup; fused: head_dim a multiple of 128 and
// scale_block of 32).  The fused kernel takes them for one token block (M <= 64).
bool stream_w8_ok(int K, int N, int head_dim, int scale_block, int num_cus, bool fused);

// MXFP8 weights -> bf16 [N, K]: out[n, k] = bf16(fp32(e4m3(codes[n, k]) * 2^(scales[n, k / 32] - 127))),
// the dequantisation rule of the table rows (K a multiple of 32).
hipError_t launch_expand_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t N, int K, uint16_t* out,
                               hipStream_t stream);

// Arguments of the tiled kernels (256-token x 256-column tiles, for large token counts).
struct TiledArgs {
  const uint16_t* wkv;  // [N, K] bf16
  // fp8 schedule (MXFP8 weights and an MXFP8 table): weight codes [N, K] and E8M0 scales
  // [N, K / 32]; the gathered rows are staged as codes [M, K] and E8M0 scales [M, K / 32]
  int mx;
  const uint8_t* wkv8;
  const uint8_t* wkv8s;
  const uint8_t* tok8;
  const uint8_t* tok8s;
  int64_t M;
  int K, N, dim;
  // projection alone
  const uint16_t* emb;  // [M, K] bf16
  uint16_t* kv;         // [M, N] bf16
  // whole forward
  const uint16_t* x;
  const int64_t* hash_ids;
  const uint8_t* token_mask;
  const uint8_t* table;
  const void* scales;  // fp32, or E8M0 bytes when scale_e8m0
  const float* q_weight;
  const float* k_weight;
  uint16_t* out;
  int32_t* err_count;
  int n_cols, head_dim, scale_block, scale_e8m0;
  int64_t n_rows;
  float eps, clamp, inv_sqrt_dim;
  uint32_t spin_budget;
  // workspace views (set by the launcher)
  void* ws;
  int n_vcb;
  size_t slot_off, part_off;
  // split K (fused schedule): tiles split_from .. tiles - 1 (at most 128) are each computed by
  // two workgroups over the two halves of K; the first to finish leaves its fp32 partial tile in
  // kpart.  split_from = tiles: no split.
  int64_t split_from;
  size_t split_off;  // per-split-tile arrival and hand-off words (control words)
  float* kpart;      // [split tile][256 x 256] fp32 (staging area)
};

// Shapes the tiled kernels take: N a multiple of 256, K of 64 (fused: also dim of 256).
bool tiled_shape_ok(int N, int K, int dim, bool fused);
// The fp8 tiled schedule (fused only): also K a multiple of 128, and the table's E8M0 scales
// covering whole 32-feature blocks (scale_block a multiple of 32).
bool tiled_mx_ok(int N, int K, int dim, int scale_block);
// Control words of the fused tiled schedule (zero before and after every call) and its staging
// area: the dequantised rows (M x K bf16) and room for the split-K partial tiles (contents
// unspecified after a call).  Neither size decreases with M.
size_t tiled_control_bytes(int64_t M, int dim);
size_t tiled_staging_bytes(int64_t M, int K, int N);
size_t tiled_staging_bytes_mx(int64_t M, int K, int N);  // rows as fp8 codes + E8M0 scales
hipError_t launch_kv_proj_tiled(const TiledArgs& a, hipStream_t stream);
// Whole forward, tiled schedule: the gather pass `g` writes the dequantised rows into `staging`
// (tiled_staging_bytes, 256-byte aligned), then the tiled kernel runs with `workspace` as its
// control words (tiled_control_bytes, zero on entry, left zero).  num_cus: compute units of the
// device (the last, partial round of tiles is split over K).
hipError_t launch_forward_tiled(TiledArgs a, const GatherArgs& g, void* workspace, void* staging, int num_cus,
                                hipStream_t stream);

}  // namespace engram
