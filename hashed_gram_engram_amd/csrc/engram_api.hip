// C ABI of libengram.so: synchronous argument checks, then kernel launches on the caller's
// stream.  No device memory is allocated here.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/engram.h"
#include "launch.h"

using namespace engram;

namespace {

constexpr uint32_t kSpinBudgetDefault = 1u << 22;  // ~1 s of sleeping polls before a wait gives up
std::atomic<uint32_t> g_spin_budget{kSpinBudgetDefault};

// From this many tokens on, the tiled schedule (256 x 256 MFMA tiles, each weight panel read
// once per 256 tokens) replaces weight streaming (all of wkv read once per 64-token block).
// The whole forward switches after one token block: with at most 128 tiles its K loop is split
// over two workgroups per tile (measured at the decode layout: 133-155 us for 96-256 tokens,
// against 139-266 us streaming two to four token blocks).  The projection alone has no
// workspace for split partials and switches at 256 tokens.
constexpr int64_t kTiledMinTokens = 256;
constexpr int64_t kTiledMinTokensFused = 65;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct DeviceInfo {
  int cus = 0;
  bool gfx950 = false;
};

// Per-device facts, queried once per device.
engram_status device_info(DeviceInfo* out) {
  static DeviceInfo cache[64];
  static bool have[64] = {false};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ENGRAM_E_HIP;
  if (!have[dev]) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ENGRAM_E_HIP;
    cache[dev].cus = prop.multiProcessorCount;
    cache[dev].gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    have[dev] = true;
  }
  *out = cache[dev];
  return cache[dev].gfx950 ? ENGRAM_OK : ENGRAM_E_DEVICE;
}

engram_status check_tokens(int64_t B, int64_t T, int64_t* M) {
  if (B < 0 || T < 0) return ENGRAM_E_SHAPE;
  if (B != 0 && T > (int64_t(1) << 40) / B) return ENGRAM_E_SHAPE;
  *M = B * T;
  return ENGRAM_OK;
}

int64_t K_of(const engram_layout* l) { return int64_t(l->n_cols) * l->head_dim; }
int64_t N_of(const engram_layout* l) { return int64_t(l->hc + 1) * l->dim; }

bool use_tiled(const engram_layout* l, int64_t M, bool fused) {
  return M >= (fused ? kTiledMinTokensFused : kTiledMinTokens) &&
         tiled_shape_ok(int(N_of(l)), int(K_of(l)), l->dim, fused);
}

bool wkv_mxfp8(const engram_layout* l) { return l->wkv_format == ENGRAM_WKV_MXFP8; }

// The layout admits the two-token-block weight-streaming kernel (bf16 weights, workgroups
// spanning at most two streams, table row ids that fit 31 bits), which then takes every
// forward of 65..128 tokens.
bool tb2_layout(const engram_layout* l, int cus) {
  const int N = int(N_of(l));
  return !wkv_mxfp8(l) && l->n_rows <= 0x7FFFFFFF && stream_rows_per_group(N, stream_grid(N, cus)) <= l->dim &&
         stream_tb2_ok(int(K_of(l)), N, l->dim, l->n_cols, l->head_dim, l->scale_block, cus);
}
bool use_tb2(const engram_layout* l, int64_t M, int cus) { return M > 64 && M <= 128 && tb2_layout(l, cus); }
// The layout admits the four-token-block kernel (bf16 weights, every workgroup the same number
// of row blocks, workgroups spanning at most two streams), which then takes every forward of
// 129..256 tokens from rows gathered into the staging area.
bool tb4_layout(const engram_layout* l, int cus) {
  const int N = int(N_of(l));
  return !wkv_mxfp8(l) && stream_rows_per_group(N, stream_grid(N, cus)) <= l->dim &&
         stream_tb4_ok(int(K_of(l)), N, l->dim, cus);
}
bool use_tb4(const engram_layout* l, int64_t M, int cus) { return M > 128 && M <= 256 && tb4_layout(l, cus); }
// the tiled schedule for the whole forward
bool use_tiled_fused(const engram_layout* l, int64_t M, int cus) {
  return use_tiled(l, M, true) && !use_tb2(l, M, cus) && !use_tb4(l, M, cus);
}

// The fused weight-streaming kernel reads MXFP8 weights itself for one token block; every other
// forward with MXFP8 weights first expands them to bf16 in the staging area.
bool forward_w8_native(const engram_layout* l, int64_t M, int cus) {
  const int N = int(N_of(l));
  return wkv_mxfp8(l) && M <= 64 && stream_w8_ok(int(K_of(l)), N, l->head_dim, l->scale_block, cus, true) &&
         stream_rows_per_group(N, stream_grid(N, cus)) <= l->dim;
}

// Workspace of engram_forward for M tokens: control words at the start (the schedule in use
// leaves them zero), then room for the staging area of the tiled schedule, which sits at the
// END of the caller's buffer.  control(M) is the larger of the two schedules' control sizes for
// every token count up to M, so it never decreases with M; neither does staging(M).  Hence for
// any two calls on one buffer (same workspace_bytes W, each with W >= control + staging), the
// control words of one never overlap the staging area of the other: the dequantised rows a
// call leaves behind never sit where a later call expects zeros.
size_t forward_control(const engram_layout* l, int64_t M, int cus) {
  const int N = int(N_of(l));
  // token counts the streaming schedules take: up to the tiled threshold (256 tokens where the
  // four-token-block kernel fits the layout, 128 where the two-token-block one does), or all of
  // them when the layout has no tiled schedule
  const bool tiled_layout = tiled_shape_ok(N, int(K_of(l)), l->dim, true);
  const int64_t cap = tb4_layout(l, cus) ? 256 : tb2_layout(l, cus) ? 128 : kTiledMinTokensFused - 1;
  const int64_t Ms = tiled_layout && M > cap ? cap : M;
  size_t c = stream_workspace_bytes(Ms, N, l->dim, stream_grid(N, cus));
  if (use_tiled_fused(l, M, cus)) {
    const size_t t = tiled_control_bytes(M, l->dim);
    c = t > c ? t : c;
  }
  return (c + 255) & ~size_t(255);
}

// The tiled schedule in fp8 (MXFP8 weights and an MXFP8 table): rows staged as codes + scales,
// weights read as they are.
bool forward_tiled_mx(const engram_layout* l, int64_t M) {
  return wkv_mxfp8(l) && l->scale_format == ENGRAM_SCALE_E8M0 && use_tiled(l, M, true) &&
         tiled_mx_ok(int(N_of(l)), int(K_of(l)), l->dim, l->scale_block);
}

// Staging area: [tiled schedule: staged rows + split partials][MXFP8 weights expanded to bf16],
// each part 256-byte aligned, plus alignment slack for its start.  Neither part decreases with M
// (the expansion is absent where a kernel reads the MXFP8 weights itself: the fused streaming
// kernel up to 64 tokens, the fp8 tiled kernel above, both with an MXFP8 table; with fp32 table
// scales only the former).
size_t forward_staging_tiled(const engram_layout* l, int64_t M, int cus) {
  // the four-token-block kernel's tokens: bf16, M rounded up to 16 (its operand order)
  if (use_tb4(l, M, cus)) return (size_t((M + 15) & ~int64_t(15)) * size_t(K_of(l)) * 2 + 255) & ~size_t(255);
  if (!use_tiled_fused(l, M, cus)) return 0;
  const size_t b = forward_tiled_mx(l, M) ? tiled_staging_bytes_mx(M, int(K_of(l)), int(N_of(l)))
                                          : tiled_staging_bytes(M, int(K_of(l)), int(N_of(l)));
  return (b + 255) & ~size_t(255);
}
size_t forward_staging_wkv(const engram_layout* l, int64_t M, int cus) {
  return wkv_mxfp8(l) && !forward_w8_native(l, M, cus) && !forward_tiled_mx(l, M)
             ? size_t(N_of(l)) * size_t(K_of(l)) * 2
             : 0;
}
size_t forward_staging(const engram_layout* l, int64_t M, int cus) {
  const size_t b = forward_staging_tiled(l, M, cus) + forward_staging_wkv(l, M, cus);
  return b > 0 ? b + 256 : 0;
}

size_t forward_workspace(const engram_layout* l, int64_t M, int cus) {
  return forward_control(l, M, cus) + forward_staging(l, M, cus);
}

// ---- the workspace of engram_forward_noalloc: a fixed device array, one copy per GPU
constexpr size_t kScratchBytes = size_t(4) << 20;

// Per device: the address of that device's copy of `scratch` (from hipGetSymbolAddress; the
// array's name in host code is not a device address) and whether it has been cleared.
struct ScratchSlot {
  void* ptr = nullptr;
  bool cleared = false;
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[64];

// Runs in front of every no-allocation forward, one workgroup: on a device's first call it
// zero-fills the scratch; later, if word 0 (wait time-outs of an earlier call) is set, the
// earlier call may have left control words set, so it zero-fills the scratch again and adds the
// time-outs to *err_count (when given).  Otherwise it only reads word 0.
__global__ __launch_bounds__(256) void k_scratch_guard(uint32_t* s, size_t n16, int first, int32_t* err_count) {
  __shared__ uint32_t timeouts;
  if (threadIdx.x == 0) timeouts = s[0];
  __syncthreads();
  const uint32_t t = timeouts;
  if (!first && t == 0u) return;
  __syncthreads();
  if (threadIdx.x == 0 && !first && err_count != nullptr) atomicAdd(err_count, int32_t(t));
  uint4* p = reinterpret_cast<uint4*>(s);
  for (size_t i = threadIdx.x; i < n16; i += blockDim.x) p[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

// The scratch array itself: file scope, one copy per GPU the library runs on, held until the
// process ends.  Host code uses it only through the per-device address above.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// This device's scratch address, looked up once per device with the device current; `dev`
// receives the device, `first` whether its scratch has not been cleared yet.
engram_status scratch_of_device(void** ptr, int* dev, bool* first) {
  if (hipGetDevice(dev) != hipSuccess || *dev < 0 || *dev >= 64) return ENGRAM_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& sl = g_scratch[*dev];
  if (sl.ptr == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ENGRAM_E_HIP;
    sl.ptr = p;
  }
  *ptr = sl.ptr;
  *first = !sl.cleared;
  return ENGRAM_OK;
}

void scratch_mark_cleared(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  g_scratch[dev].cleared = true;
}

// The synchronous checks engram_forward makes of its tensor pointers.
engram_status check_forward_pointers(const uint16_t* x, const int64_t* hash_ids, const uint8_t* table,
                                     const void* scales, const void* wkv, const float* q_weight,
                                     const float* k_weight, const uint16_t* out) {
  if (!x || !hash_ids || !table || !scales || !wkv || !q_weight || !k_weight || !out) return ENGRAM_E_NULL;
  if (!aligned16(x) || !aligned16(table) || !aligned16(wkv) || !aligned16(q_weight) || !aligned16(k_weight) ||
      !aligned16(out) || (reinterpret_cast<uintptr_t>(scales) & 3u) || (reinterpret_cast<uintptr_t>(hash_ids) & 7u))
    return ENGRAM_E_ALIGN;
  return ENGRAM_OK;
}

}  // namespace

extern "C" {

const char* engram_status_str(engram_status s) {
  switch (s) {
    case ENGRAM_OK: return "ok";
    case ENGRAM_E_NULL: return "a required pointer is NULL";
    case ENGRAM_E_LAYOUT: return "invalid layout";
    case ENGRAM_E_SHAPE: return "invalid token count";
    case ENGRAM_E_ALIGN: return "tensor pointer not aligned as required";
    case ENGRAM_E_WORKSPACE: return "workspace missing or too small";
    case ENGRAM_E_HIP: return "HIP runtime error";
    case ENGRAM_E_DEVICE: return "current device is not gfx950";
    case ENGRAM_E_TIMEOUT: return "a cross-workgroup wait of engram_forward timed out (outputs are wrong)";
  }
  return "unknown status";
}

uint32_t engram_set_spin_budget(uint32_t polls) {
  return g_spin_budget.exchange(polls == 0 ? kSpinBudgetDefault : polls);
}

engram_status engram_forward_check(void* workspace, size_t workspace_bytes, engram_stream_t stream) {
  if (workspace == nullptr) return ENGRAM_E_NULL;
  if (workspace_bytes < 4 || !aligned16(workspace)) return ENGRAM_E_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return ENGRAM_E_HIP;
  uint32_t timeouts = 0;
  if (hipMemcpy(&timeouts, workspace, 4, hipMemcpyDeviceToHost) != hipSuccess) return ENGRAM_E_HIP;
  if (timeouts == 0) return ENGRAM_OK;
  if (hipMemsetAsync(workspace, 0, workspace_bytes, st) != hipSuccess) return ENGRAM_E_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return ENGRAM_E_HIP;
  return ENGRAM_E_TIMEOUT;
}

engram_status engram_layout_check(const engram_layout* l) {
  if (l == nullptr) return ENGRAM_E_NULL;
  if (l->hc != 4) return ENGRAM_E_LAYOUT;
  if (l->dim <= 0 || l->dim % 64 != 0 || l->dim > (1 << 22)) return ENGRAM_E_LAYOUT;
  if (l->n_cols <= 0 || l->head_dim <= 0 || l->head_dim % 64 != 0) return ENGRAM_E_LAYOUT;
  if (l->scale_block <= 0 || l->scale_block % 16 != 0 || l->head_dim % l->scale_block != 0)
    return ENGRAM_E_LAYOUT;
  if ((int64_t(l->n_cols) * l->head_dim) % 128 != 0) return ENGRAM_E_LAYOUT;
  if (int64_t(l->n_cols) * l->head_dim > (int64_t(1) << 20)) return ENGRAM_E_LAYOUT;
  if (l->n_rows <= 0) return ENGRAM_E_LAYOUT;
  if (l->scale_format != ENGRAM_SCALE_FP32 && l->scale_format != ENGRAM_SCALE_E8M0) return ENGRAM_E_LAYOUT;
  if (l->wkv_format != ENGRAM_WKV_BF16 && l->wkv_format != ENGRAM_WKV_MXFP8) return ENGRAM_E_LAYOUT;
  // E8M0 scales of a row are whole dwords (the streaming kernel copies them dword-wise)
  if (l->scale_format == ENGRAM_SCALE_E8M0 && (l->head_dim / l->scale_block) % 4 != 0) return ENGRAM_E_LAYOUT;
  if (!(l->eps >= 0.0f) || !isfinite(l->eps) || !(l->clamp >= 0.0f) || !isfinite(l->clamp))
    return ENGRAM_E_LAYOUT;
  return ENGRAM_OK;
}

engram_status engram_param_counts(const engram_layout* l, int64_t out[3]) {
  engram_status st = engram_layout_check(l);
  if (st != ENGRAM_OK) return st;
  if (out == nullptr) return ENGRAM_E_NULL;
  out[0] = l->n_rows * l->head_dim;
  out[1] = K_of(l) * N_of(l);
  out[2] = int64_t(2) * l->hc * l->dim;
  return ENGRAM_OK;
}

size_t engram_forward_workspace_bytes(const engram_layout* l, int64_t B, int64_t T) {
  if (engram_layout_check(l) != ENGRAM_OK) return 0;
  int64_t M = 0;
  if (check_tokens(B, T, &M) != ENGRAM_OK) return 0;
  DeviceInfo di;
  int cus = (device_info(&di) == ENGRAM_OK) ? di.cus : 256;
  return forward_workspace(l, M, cus);
}

size_t engram_forward_staging_bytes(const engram_layout* l, int64_t B, int64_t T) {
  if (engram_layout_check(l) != ENGRAM_OK) return 0;
  int64_t M = 0;
  if (check_tokens(B, T, &M) != ENGRAM_OK) return 0;
  DeviceInfo di;
  int cus = (device_info(&di) == ENGRAM_OK) ? di.cus : 256;
  return forward_staging(l, M, cus);
}

engram_status engram_gather_dequant(const engram_layout* l, const uint8_t* table, const void* scales,
                                    const int64_t* hash_ids, int64_t B, int64_t T, uint16_t* emb,
                                    int32_t* err_count, engram_stream_t stream) {
  engram_status st = engram_layout_check(l);
  if (st != ENGRAM_OK) return st;
  int64_t M = 0;
  if ((st = check_tokens(B, T, &M)) != ENGRAM_OK) return st;
  if (M == 0) return ENGRAM_OK;
  if (!table || !scales || !hash_ids || !emb) return ENGRAM_E_NULL;
  if (!aligned16(table) || !aligned16(emb) || (reinterpret_cast<uintptr_t>(scales) & 3u) ||
      (reinterpret_cast<uintptr_t>(hash_ids) & 7u))
    return ENGRAM_E_ALIGN;
  DeviceInfo di;
  if ((st = device_info(&di)) != ENGRAM_OK) return st;
  GatherArgs a{table, scales, hash_ids, M * l->n_cols, l->head_dim, l->scale_block,
               l->scale_format == ENGRAM_SCALE_E8M0, l->n_rows, emb, err_count};
  return launch_gather_dequant(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? ENGRAM_OK
                                                                                        : ENGRAM_E_HIP;
}

engram_status engram_kv_proj(const engram_layout* l, const uint16_t* emb, const void* wkv, int64_t B,
                             int64_t T, uint16_t* kv, engram_stream_t stream) {
  engram_status st = engram_layout_check(l);
  if (st != ENGRAM_OK) return st;
  int64_t M = 0;
  if ((st = check_tokens(B, T, &M)) != ENGRAM_OK) return st;
  if (M == 0) return ENGRAM_OK;
  if (!emb || !wkv || !kv) return ENGRAM_E_NULL;
  if (!aligned16(emb) || !aligned16(wkv) || !aligned16(kv)) return ENGRAM_E_ALIGN;
  DeviceInfo di;
  if ((st = device_info(&di)) != ENGRAM_OK) return st;
  if (wkv_mxfp8(l)) {
    // MXFP8 weights: the weight-streaming kernel for every token count
    if (!stream_w8_ok(int(K_of(l)), int(N_of(l)), l->head_dim, l->scale_block, di.cus, false)) return ENGRAM_E_LAYOUT;
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    a.w8 = 1;
    a.wkv8 = static_cast<const uint8_t*>(wkv);
    a.wkv8s = a.wkv8 + size_t(N_of(l)) * size_t(K_of(l));
    a.M = M;
    a.K = int(K_of(l));
    a.N = int(N_of(l));
    a.dim = l->dim;
    a.emb = emb;
    a.kv = kv;
    return launch_kv_proj_stream(a, di.cus, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? ENGRAM_OK
                                                                                                  : ENGRAM_E_HIP;
  }
  const uint16_t* wkv16 = static_cast<const uint16_t*>(wkv);
  if (use_tiled(l, M, false)) {
    TiledArgs a;
    memset(&a, 0, sizeof(a));
    a.wkv = wkv16;
    a.M = M;
    a.K = int(K_of(l));
    a.N = int(N_of(l));
    a.dim = l->dim;
    a.emb = emb;
    a.kv = kv;
    return launch_kv_proj_tiled(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? ENGRAM_OK
                                                                                         : ENGRAM_E_HIP;
  }
  StreamArgs a;
  memset(&a, 0, sizeof(a));
  a.wkv = wkv16;
  a.M = M;
  a.K = int(K_of(l));
  a.N = int(N_of(l));
  a.dim = l->dim;
  a.emb = emb;
  a.kv = kv;
  return launch_kv_proj_stream(a, di.cus, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? ENGRAM_OK
             : ENGRAM_E_HIP;
}

engram_status engram_hash_ids(const engram_hash_layout* hl, const uint32_t* token_map,
                              const int64_t* multipliers, const int64_t* primes,
                              const int64_t* offsets, const int64_t* input_ids,
                              const uint8_t* token_mask, int64_t B, int64_t L, int64_t start_pos,
                              int64_t* history, int64_t* hash_ids, int32_t* err_count,
                              engram_stream_t stream) {
  if (hl == nullptr) return ENGRAM_E_NULL;
  if (hl->n_layers < 1 || hl->max_ngram < 2 || hl->max_ngram > 8 || hl->n_heads < 1 || hl->vocab < 1 ||
      hl->history_len < 1 || int64_t(hl->n_layers) * (hl->max_ngram - 1) * hl->n_heads > (1 << 20))
    return ENGRAM_E_LAYOUT;
  if (B < 0 || L < 0 || start_pos < 0) return ENGRAM_E_SHAPE;
  if (B > 0 && L > (int64_t(1) << 40) / B) return ENGRAM_E_SHAPE;
  if (start_pos + L > hl->history_len) return ENGRAM_E_SHAPE;
  if (B * L == 0) return ENGRAM_OK;
  if (!token_map || !multipliers || !primes || !offsets || !input_ids || !history || !hash_ids)
    return ENGRAM_E_NULL;
  if ((reinterpret_cast<uintptr_t>(token_map) & 3u) || (reinterpret_cast<uintptr_t>(multipliers) & 7u) ||
      (reinterpret_cast<uintptr_t>(primes) & 7u) || (reinterpret_cast<uintptr_t>(offsets) & 7u) ||
      (reinterpret_cast<uintptr_t>(input_ids) & 7u) || (reinterpret_cast<uintptr_t>(history) & 7u) ||
      (reinterpret_cast<uintptr_t>(hash_ids) & 7u))
    return ENGRAM_E_ALIGN;
  engram_status st;
  DeviceInfo di;
  if ((st = device_info(&di)) != ENGRAM_OK) return st;
  HashArgs a;
  memset(&a, 0, sizeof(a));
  a.token_map = token_map;
  a.multipliers = multipliers;
  a.primes = primes;
  a.offsets = offsets;
  a.input_ids = input_ids;
  a.token_mask = token_mask;
  a.history = history;
  a.hash_ids = hash_ids;
  a.err_count = err_count;
  a.B = B;
  a.L = L;
  a.start_pos = start_pos;
  a.vocab = hl->vocab;
  a.history_len = hl->history_len;
  a.n_layers = hl->n_layers;
  a.max_ngram = hl->max_ngram;
  a.n_heads = hl->n_heads;
  a.pad_id = hl->pad_id;
  return launch_hash_ids(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? ENGRAM_OK : ENGRAM_E_HIP;
}

engram_status engram_gate_apply(const engram_layout* l, const uint16_t* x, const uint16_t* kv,
                                const float* q_weight, const float* k_weight, const uint8_t* token_mask,
                                int64_t B, int64_t T, uint16_t* out, float* gate, engram_stream_t stream) {
  engram_status st = engram_layout_check(l);
  if (st != ENGRAM_OK) return st;
  int64_t M = 0;
  if ((st = check_tokens(B, T, &M)) != ENGRAM_OK) return st;
  if (M == 0) return ENGRAM_OK;
  if (!x || !kv || !q_weight || !k_weight || !out) return ENGRAM_E_NULL;
  if (!aligned16(x) || !aligned16(kv) || !aligned16(q_weight) || !aligned16(k_weight) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(gate) & 3u))
    return ENGRAM_E_ALIGN;
  if (M > 0x7FFFFFFF) return ENGRAM_E_SHAPE;
  DeviceInfo di;
  if ((st = device_info(&di)) != ENGRAM_OK) return st;
  GateArgs a{x, kv, q_weight, k_weight, token_mask, M, l->dim, l->eps, l->clamp,
             float(1.0 / sqrt(double(l->dim))), out, gate};
  return launch_gate_apply(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? ENGRAM_OK : ENGRAM_E_HIP;
}

engram_status engram_forward(const engram_layout* l, const uint16_t* x, const int64_t* hash_ids,
                             const uint8_t* token_mask, const uint8_t* table, const void* scales,
                             const void* wkv_arg, const float* q_weight, const float* k_weight, int64_t B,
                             int64_t T, uint16_t* out, void* workspace, size_t workspace_bytes,
                             int32_t* err_count, engram_stream_t stream) {
  engram_status st = engram_layout_check(l);
  if (st != ENGRAM_OK) return st;
  int64_t M = 0;
  if ((st = check_tokens(B, T, &M)) != ENGRAM_OK) return st;
  if (M == 0) return ENGRAM_OK;
  if ((st = check_forward_pointers(x, hash_ids, table, scales, wkv_arg, q_weight, k_weight, out)) != ENGRAM_OK)
    return st;
  DeviceInfo di;
  if ((st = device_info(&di)) != ENGRAM_OK) return st;
  const int N = int(N_of(l));
  const size_t need = forward_workspace(l, M, di.cus);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return ENGRAM_E_WORKSPACE;
  // the staging area: the last forward_staging() bytes of the buffer, 256-byte aligned
  const size_t stg = forward_staging(l, M, di.cus);
  const uintptr_t stg_start =
      (reinterpret_cast<uintptr_t>(workspace) + workspace_bytes - stg + 255) & ~uintptr_t(255);
  const bool native8 = forward_w8_native(l, M, di.cus);
  const bool tiled8 = forward_tiled_mx(l, M);
  const uint16_t* wkv = static_cast<const uint16_t*>(wkv_arg);
  if (wkv_mxfp8(l) && !native8 && !tiled8) {
    // MXFP8 weights for a bf16 schedule: expand them behind the tiled part of the staging area
    uint16_t* copy = reinterpret_cast<uint16_t*>(stg_start + forward_staging_tiled(l, M, di.cus));
    const uint8_t* codes = static_cast<const uint8_t*>(wkv_arg);
    if (launch_expand_mxfp8(codes, codes + size_t(N) * size_t(K_of(l)), N, int(K_of(l)), copy,
                            reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
      return ENGRAM_E_HIP;
    wkv = copy;
  }
  if (use_tiled_fused(l, M, di.cus)) {
    TiledArgs a;
    memset(&a, 0, sizeof(a));
    a.wkv = wkv;
    if (tiled8) {
      a.mx = 1;
      a.wkv8 = static_cast<const uint8_t*>(wkv_arg);
      a.wkv8s = a.wkv8 + size_t(N) * size_t(K_of(l));
    }
    a.M = M;
    a.K = int(K_of(l));
    a.N = N;
    a.dim = l->dim;
    a.x = x;
    a.hash_ids = hash_ids;
    a.token_mask = token_mask;
    a.table = table;
    a.scales = scales;
    a.q_weight = q_weight;
    a.k_weight = k_weight;
    a.out = out;
    a.err_count = err_count;
    a.n_cols = l->n_cols;
    a.head_dim = l->head_dim;
    a.scale_block = l->scale_block;
    a.scale_e8m0 = l->scale_format == ENGRAM_SCALE_E8M0;
    a.n_rows = l->n_rows;
    a.eps = l->eps;
    a.clamp = l->clamp;
    a.inv_sqrt_dim = float(1.0 / sqrt(double(l->dim)));
    a.spin_budget = g_spin_budget.load(std::memory_order_relaxed);
    GatherArgs g{table, scales, hash_ids, M * l->n_cols, l->head_dim, l->scale_block,
                 l->scale_format == ENGRAM_SCALE_E8M0, l->n_rows, nullptr, err_count};
    return launch_forward_tiled(a, g, workspace, reinterpret_cast<void*>(stg_start), di.cus,
                                reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? ENGRAM_OK
               : ENGRAM_E_HIP;
  }
  const int G = stream_grid(N, di.cus);
  if (stream_rows_per_group(N, G) > l->dim) return ENGRAM_E_LAYOUT;  // a workgroup spans <= 2 segments
  StreamArgs a;
  memset(&a, 0, sizeof(a));
  a.wkv = wkv;
  if (native8) {
    a.w8 = 1;
    a.wkv8 = static_cast<const uint8_t*>(wkv_arg);
    a.wkv8s = a.wkv8 + size_t(N) * size_t(K_of(l));
  }
  a.M = M;
  a.K = int(K_of(l));
  a.N = N;
  a.dim = l->dim;
  a.x = x;
  a.hash_ids = hash_ids;
  a.token_mask = token_mask;
  a.table = table;
  a.scales = scales;
  a.q_weight = q_weight;
  a.k_weight = k_weight;
  a.out = out;
  a.err_count = err_count;
  a.n_cols = l->n_cols;
  a.head_dim = l->head_dim;
  a.scale_block = l->scale_block;
  a.scale_e8m0 = l->scale_format == ENGRAM_SCALE_E8M0;
  a.n_rows = l->n_rows;
  a.eps = l->eps;
  a.clamp = l->clamp;
  a.inv_sqrt_dim = float(1.0 / sqrt(double(l->dim)));
  a.spin_budget = g_spin_budget.load(std::memory_order_relaxed);
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (use_tb4(l, M, di.cus)) {
    // the rows gathered and dequantised into the staging area (in the MFMA operand order), then
    // one pass over the weights
    uint16_t* emb = reinterpret_cast<uint16_t*>(stg_start);
    GatherArgs g{table, scales, hash_ids, M * l->n_cols, l->head_dim, l->scale_block,
                 l->scale_format == ENGRAM_SCALE_E8M0, l->n_rows, emb, err_count, l->n_cols,
                 ((M + 15) & ~int64_t(15)) * l->n_cols};
    e = launch_gather_dequant(g, hs);
    a.emb = emb;
    if (e == hipSuccess) e = launch_forward_tb4(a, workspace, di.cus, hs);
  } else if (use_tb2(l, M, di.cus)) {
    e = launch_forward_tb2(a, workspace, di.cus, hs);
  } else {
    e = launch_forward_stream(a, workspace, di.cus, hs);
  }
  return e == hipSuccess ? ENGRAM_OK : ENGRAM_E_HIP;
}

engram_status engram_forward_noalloc(const engram_layout* l, const uint16_t* x, const int64_t* hash_ids,
                                     const uint8_t* token_mask, const uint8_t* table, const void* scales,
                                     const void* wkv, const float* q_weight, const float* k_weight, int64_t B,
                                     int64_t T, uint16_t* out, int32_t* err_count, engram_stream_t stream) {
  engram_status st = engram_layout_check(l);
  if (st != ENGRAM_OK) return st;
  int64_t M = 0;
  if ((st = check_tokens(B, T, &M)) != ENGRAM_OK) return st;
  if (M == 0) return ENGRAM_OK;
  if ((st = check_forward_pointers(x, hash_ids, table, scales, wkv, q_weight, k_weight, out)) != ENGRAM_OK)
    return st;
  DeviceInfo di;
  if ((st = device_info(&di)) != ENGRAM_OK) return st;
  if (forward_workspace(l, M, di.cus) > kScratchBytes) return ENGRAM_E_WORKSPACE;
  void* ptr = nullptr;
  int dev = 0;
  bool first = false;
  if ((st = scratch_of_device(&ptr, &dev, &first)) != ENGRAM_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_scratch_guard, dim3(1), dim3(256), 0, hs, static_cast<uint32_t*>(ptr), kScratchBytes / 16,
                     first ? 1 : 0, err_count);
  if (hipGetLastError() != hipSuccess) return ENGRAM_E_HIP;
  if (first) scratch_mark_cleared(dev);
  return engram_forward(l, x, hash_ids, token_mask, table, scales, wkv, q_weight, k_weight, B, T, out, ptr,
                        kScratchBytes, err_count, stream);
}

}  // extern "C"
