/* engram.h: C ABI of the MI355X (gfx950) Engram forward library, libengram.so.
 *
 * The operation is the Engram block of DeepSeek-V4.1-Flash as given on the
 * "DeepSeek-V4.1 / blocks / engram-second" page (code panel: Engram.forward and
 * ParallelEngramEmbedding.forward), with the tensor statement of that page:
 * x [B, T, hc, dim] in, the same shape out, hash_ids [B, T, n_cols] global row ids.
 *
 * Conventions shared by every entry point:
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - Every tensor pointer is a DEVICE pointer to a contiguous row-major tensor, 16-byte
 *    aligned.  The caller owns every buffer; the library allocates no device memory and
 *    keeps no state between calls (beyond the caller-owned workspace of engram_forward).
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream).  Arguments are
 *    checked synchronously on the host first; on any error nothing is enqueued and a
 *    negative status is returned.  B * T == 0 is a no-op returning ENGRAM_OK.
 *  - hc must be 4; dim a multiple of 64 and at most 2^22; head_dim a multiple of 64 and of scale_block;
 *    scale_block a multiple of 16; n_cols * head_dim a multiple of 128.
 *  - Hash ids outside [0, n_rows) read as an all-zero row (a single-shard
 *    ParallelEngramEmbedding zero-fills rows it does not hold); when err_count is not NULL
 *    each such (token, column) pair adds 1 to *err_count (device int32), so a caller can
 *    check after synchronising.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* engram_stream_t; /* a hipStream_t */

typedef enum {
  ENGRAM_OK = 0,
  ENGRAM_E_NULL = -1,      /* a required pointer is NULL                        */
  ENGRAM_E_LAYOUT = -2,    /* the layout violates a constraint listed above      */
  ENGRAM_E_SHAPE = -3,     /* negative B or T, or a size that overflows          */
  ENGRAM_E_ALIGN = -4,     /* a tensor pointer is not aligned as required        */
  ENGRAM_E_WORKSPACE = -5, /* workspace missing or smaller than required         */
  ENGRAM_E_HIP = -6,       /* the HIP runtime refused a launch or query          */
  ENGRAM_E_DEVICE = -7,    /* the current device is not gfx950                   */
  ENGRAM_E_TIMEOUT = -8    /* a cross-workgroup wait of engram_forward gave up: the outputs of
                              the calls since the last engram_forward_check are wrong         */
} engram_status;

/* Block scales of the fp8 table: one fp32 value per block, or one E8M0 byte per block (the
 * MXFP8 format of the official tables, "Engram in DeepSeek V4.1 Flash", Step 2: OCP MX v1.0
 * scale, value 2^(e - 127), 0xFF = NaN). */
typedef enum { ENGRAM_SCALE_FP32 = 0, ENGRAM_SCALE_E8M0 = 1 } engram_scale_format;

/* Storage of the wkv projection.  BF16: [(hc + 1) * dim, K] bf16, the Linear weight.  MXFP8: the
 * same matrix as e4m3fn codes with one E8M0 scale per 32 consecutive input features, in ONE
 * buffer: codes [(hc + 1) * dim, K] uint8, immediately followed by scales [(hc + 1) * dim, K / 32]
 * uint8 (N * K * 33 / 32 bytes).  Weight (n, k) is bf16(fp32(e4m3(code[n, k]) * 2^(scale[n, k / 32]
 * - 127))), the table rows' rule, so the projection is that of the bf16 matrix of these values.
 * (The pages state that the projections are stored in FP8 ("DeepSeek's Other Modules", Engram)
 * without their scale layout; this one is the MX layout of the tables along the input features.) */
typedef enum { ENGRAM_WKV_BF16 = 0, ENGRAM_WKV_MXFP8 = 1 } engram_wkv_format;

/* Sizes of one Engram instance (engram-second page, Engram.__init__ and config.json:
 * hc_mult = 4, dim = 5120, n_hash_cols = (engram_max_ngram_size - 1) * engram_n_heads = 24,
 * engram_head_dim = 256, norm_eps = 1e-20, clamp value 1e-6).  scale_block is the number of
 * features sharing one dequantisation scale (32 on the pages, 128 in the large synthetic
 * workloads); scale_format is an engram_scale_format (E8M0 needs head_dim / scale_block to be
 * a multiple of 4, e.g. 256 / 32). */
typedef struct {
  int32_t hc;
  int32_t dim;
  int32_t n_cols;
  int32_t head_dim;
  int32_t scale_block;
  int32_t scale_format; /* engram_scale_format */
  int32_t wkv_format;   /* engram_wkv_format */
  int64_t n_rows;   /* rows of the table: the sum of the prime range lengths */
  float eps;
  float clamp;
} engram_layout;

/* Host-only checks of a layout; no device work. */
engram_status engram_layout_check(const engram_layout* layout);

/* Learned element counts of one instance (engram-second page, Parameters table):
 * out[0] = table entries n_rows * head_dim, out[1] = wkv entries
 * (n_cols * head_dim) * ((hc + 1) * dim), out[2] = gate weights 2 * hc * dim. */
engram_status engram_param_counts(const engram_layout* layout, int64_t out[3]);

/* Bytes of workspace engram_forward needs for B x T tokens on the current device (0 on an
 * invalid layout).  The workspace holds control words at its start (counters, gate slots,
 * partial sums and, for up to four 64-token blocks, the bf16 value tiles that the weight-streaming
 * kernels hand to their apply workgroups) and, for token counts where the tiled schedule or the
 * four-token-block streaming kernel runs, a staging area for the dequantised rows in its last
 * engram_forward_staging_bytes() bytes.  It must be zero-filled
 * before its first use.  Every call leaves all control words zero again; the staging area's
 * contents are unspecified after a call.  So one workspace serves any number of calls with one
 * layout and any B x T it is large enough for, on one stream without clearing, provided every
 * call on it passes the same workspace_bytes (neither part shrinks as B x T grows, so the
 * control words of any call then lie below the staging area of every other).  The exception is word 0, which counts cross-workgroup waits
 * that timed out (0 in correct operation); engram_forward_check reports it and zero-fills the
 * workspace after a time-out.  Calls that overlap in time must use different workspaces. */
size_t engram_forward_workspace_bytes(const engram_layout* layout, int64_t B, int64_t T);

/* Bytes at the end of the workspace that engram_forward uses as a staging area for B x T
 * tokens: the dequantised rows (B x T x n_cols x head_dim bf16), room for the fp32 partial
 * tiles of a K loop split over two workgroups (taken for every tile when a call has few tiles,
 * else for the tiles of a last, partial round; a fixed 32 MB per layout), alignment slack; 0
 * where the fused weight-streaming schedules of one or two token blocks run (up to 64 tokens,
 * and 65..128 with bf16 weights where the layout admits them), which keep the rows on chip.
 * Where the four-token-block streaming kernel runs (129..256 tokens, bf16 weights, layouts
 * whose streaming workgroups own equal row counts) only the rows, B x T rounded up to 16.  With
 * MXFP8 weights and an MXFP8 table the rows are staged as fp8 codes plus one E8M0 byte per 32
 * features (K + K / 32 bytes per token); with MXFP8 weights and fp32 table scales above 64 tokens (or on shapes the
 * streaming kernel does not take) the weights are expanded to bf16 there as well (N x K x 2
 * bytes).  Included in engram_forward_workspace_bytes(). */
size_t engram_forward_staging_bytes(const engram_layout* layout, int64_t B, int64_t T);

/* S1 + S2: row gather and dequantisation (engram-second page,
 * ParallelEngramEmbedding.forward, single shard; flatten as in Engram.forward).
 *   table    [n_rows, head_dim]   uint8  fp8 e4m3fn codes
 *   scales   [n_rows, head_dim / scale_block] fp32, or uint8 E8M0 exponents (scale_format);
 *            4-byte aligned
 *   hash_ids [B, T, n_cols]       int64  global row ids
 *   emb      [B, T, n_cols * head_dim] bf16 out:
 *            emb[m, j * head_dim + c] = bf16(fp32(e4m3(table[r, c]) * scale(r, c / scale_block)))
 *            with r = hash_ids[m, j]; rounding to nearest even; NaN is written as 0x7FC0. */
engram_status engram_gather_dequant(const engram_layout* layout, const uint8_t* table,
                                    const void* scales, const int64_t* hash_ids, int64_t B,
                                    int64_t T, uint16_t* emb, int32_t* err_count,
                                    engram_stream_t stream);

/* S3: the wkv projection (engram-second page, self.wkv, a Linear from n_cols * head_dim to
 * (hc + 1) * dim features):
 *   emb [B, T, K] bf16 with K = n_cols * head_dim
 *   wkv [(hc + 1) * dim, K] bf16 (Linear weight layout [out, in]), or the MXFP8 buffer of
 *       layout->wkv_format (then K / 4 must be a multiple of 128 and the weight-streaming
 *       schedule must give every compute unit 1 to 8 blocks of 16 rows, as at the model's
 *       25,600 rows on 256 compute units, else ENGRAM_E_LAYOUT)
 *   kv  [B, T, (hc + 1) * dim] bf16 out: kv[m, n] = bf16(sum_k emb[m, k] * wkv[n, k]),
 *       fp32 accumulation, rounded to nearest even.  Columns [s * dim, (s + 1) * dim) are
 *       the key of stream s; the last dim columns are the shared value. */
engram_status engram_kv_proj(const engram_layout* layout, const uint16_t* emb,
                             const void* wkv, int64_t B, int64_t T, uint16_t* kv,
                             engram_stream_t stream);

/* S4 - S6: gate and residual add from a given kv (engram-second page, Engram.forward after
 * the projection; zhuai.tech "Step 3: Inject memory at the correct layer boundary"):
 *   x          [B, T, hc, dim] bf16
 *   kv         [B, T, (hc + 1) * dim] bf16
 *   q_weight, k_weight [hc, dim] fp32 (used only as their fp32 product)
 *   token_mask [B, T] uint8, 0 = closed (the token passes through bit for bit), NULL = all open
 *   out        [B, T, hc, dim] bf16; may be the same pointer as x (in place)
 *   gate       [B, T, hc] fp32 out, may be NULL
 * Per (token, stream s): rstd = rsqrt(mean(h^2) + eps) * rsqrt(mean(key_s^2) + eps),
 * dot = sum(h * q * k * key_s) * rstd / sqrt(dim),
 * g = sigmoid(copysign(sqrt(max(|dot|, clamp)), dot)), out = bf16(h + g * value). */
engram_status engram_gate_apply(const engram_layout* layout, const uint16_t* x,
                                const uint16_t* kv, const float* q_weight,
                                const float* k_weight, const uint8_t* token_mask, int64_t B,
                                int64_t T, uint16_t* out, float* gate, engram_stream_t stream);

/* The whole Engram forward in one call (engram-second page, Engram.forward): S1 - S6 with
 * the arguments above (wkv in either format of layout->wkv_format).  Key and value stay on chip; only small per-tile partial sums pass
 * through `workspace` (engram_forward_workspace_bytes), and at large token counts the
 * dequantised rows pass through its staging area.  out may equal x.  Results equal
 * engram_gate_apply(engram_kv_proj(engram_gather_dequant(...))) up to the summation order of
 * the gate reductions. */
engram_status engram_forward(const engram_layout* layout, const uint16_t* x,
                             const int64_t* hash_ids, const uint8_t* token_mask,
                             const uint8_t* table, const void* scales, const void* wkv,
                             const float* q_weight, const float* k_weight, int64_t B, int64_t T,
                             uint16_t* out, void* workspace, size_t workspace_bytes,
                             int32_t* err_count, engram_stream_t stream);

/* engram_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation and results, with
 * no workspace argument.  The workspace is a fixed array of the library, `scratch`, 4 MiB per GPU
 * (a static device array: each GPU the library runs on holds its own copy until the process
 * ends); that covers calls of up to 128 tokens at the model's layout (the fused weight-streaming
 * schedules); a call that needs more returns ENGRAM_E_WORKSPACE before anything is enqueued.
 * Nothing is allocated, here or in the kernels.  Each call first enqueues a one-workgroup guard
 * kernel: on a GPU's first call it zero-fills the scratch; later it reads the scratch's time-out
 * word and, if an earlier call's wait timed out (its outputs were wrong), zero-fills the scratch
 * again and adds the time-outs to *err_count (when err_count is not NULL).  All calls on one GPU
 * share its scratch: calls that overlap in time on one GPU (different streams, host threads)
 * race and give wrong results; serialise them.  Other arguments as engram_forward. */
engram_status engram_forward_noalloc(const engram_layout* layout, const uint16_t* x,
                                     const int64_t* hash_ids, const uint8_t* token_mask,
                                     const uint8_t* table, const void* scales, const void* wkv,
                                     const float* q_weight, const float* k_weight, int64_t B,
                                     int64_t T, uint16_t* out, int32_t* err_count,
                                     engram_stream_t stream);

/* Reports whether the engram_forward calls that used `workspace` since the last check ran
 * correctly.  The fused schedules hand partial sums and gates between workgroups of one launch
 * through the workspace; a workgroup waits for a hand-off only on work of lower-numbered
 * workgroups that never waits itself, which is deadlock-free because the hardware dispatches a
 * launch's workgroups in increasing order (every workgroup that is waited on has started before
 * the wait, and finishes since it waits for nothing).  Each wait is still bounded (about a second
 * of polling, see engram_set_spin_budget); a wait that gives up counts itself in workspace word 0
 * and the call's outputs are then wrong.
 * This call waits for `stream` (hipStreamSynchronize), reads word 0, and returns ENGRAM_OK if it
 * is zero.  Otherwise it zero-fills the whole workspace (a late hand-off may have left control
 * words set) on `stream`, waits for that, and returns ENGRAM_E_TIMEOUT; the workspace is then
 * ready for further calls.  It cannot be recorded into a graph (it synchronises). */
engram_status engram_forward_check(void* workspace, size_t workspace_bytes, engram_stream_t stream);

/* Bound of every cross-workgroup wait of engram_forward, in polls (each a short sleep): 0
 * restores the default (2^22 polls, about a second).  Process-wide; applies to launches made
 * after the call; returns the previous bound.  A small bound makes waits give up early, which is
 * how a caller (a test) can drive the time-out path while every kernel still exits normally. */
uint32_t engram_set_spin_budget(uint32_t polls);

/* The hash step in front of the path (engram-second page, code panel, the hash module's
 * forward; "DeepSeek's Other Modules", Engram, The lookup pipeline): raw token ids -> the
 * n_cols = (max_ngram - 1) * n_heads global row ids of every Engram layer.  The model's values:
 * n_layers = 2 (layers 1 and 14), max_ngram = 4 (2-, 3- and 4-grams), n_heads = 8, pad_id = 2,
 * vocab = 129,280 (config.json). */
typedef struct {
  int32_t n_layers;
  int32_t max_ngram;   /* 2 .. 8 */
  int32_t n_heads;
  int32_t pad_id;      /* compressed id read for a look-back before the start or past a dead token */
  int64_t vocab;       /* entries of the token map */
  int64_t history_len; /* positions per sequence the history holds */
} engram_hash_layout;

/* Per position p = start_pos + l of sequence b: compressed = token_map[input_ids[b, l]], or
 * dead (-1) where token_mask is 0 (image spans) or the id lies outside [0, vocab) (counted in
 * *err_count).  Look-back s (0 <= s < max_ngram) takes the compressed id of position p - s (this
 * call's tokens, or history[b, p - s] for earlier positions); from the first look-back that lies
 * before position 0 or is dead on, it takes pad_id.  For layer y the products t_s *
 * multipliers[y, s] wrap modulo 2^64 (two's complement int64, as the page's tensors); their
 * running XOR over s = 0..n is the (n+1)-gram hash h_n, and column (n - 1) * n_heads + k is
 * floor_mod(h_n, primes[y, n - 1, k]) + offsets[y, column].
 *   token_map   [vocab] uint32       compressed ids
 *   multipliers [n_layers, max_ngram] int64 (odd on the pages)
 *   primes      [n_layers, max_ngram - 1, n_heads] int64 > 0 (a non-positive prime writes -1
 *               and counts an error)
 *   offsets     [n_layers, n_cols] int64
 *   input_ids   [B, L] int64; token_mask [B, L] uint8 or NULL (all live)
 *   history     [B, history_len] int64 in/out: compressed ids of positions < start_pos from
 *               earlier calls; this call writes positions start_pos .. start_pos + L - 1.
 *               Requires start_pos + L <= history_len.  Chunked calls over a sequence give the
 *               row ids of one call over the whole of it.
 *   hash_ids    [n_layers, B, L, n_cols] int64 out, layer-major (the page returns
 *               [B, L, n_layers, n_cols]): each layer's [B, L, n_cols] slice is contiguous, the
 *               hash_ids argument of engram_forward for that layer's module. */
engram_status engram_hash_ids(const engram_hash_layout* layout, const uint32_t* token_map,
                              const int64_t* multipliers, const int64_t* primes,
                              const int64_t* offsets, const int64_t* input_ids,
                              const uint8_t* token_mask, int64_t B, int64_t L, int64_t start_pos,
                              int64_t* history, int64_t* hash_ids, int32_t* err_count,
                              engram_stream_t stream);

/* Static description of a status code. */
const char* engram_status_str(engram_status status);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
