// C ABI of libengram.so: synchronous argument checks, then kernel launches on the caller's
// stream.  No device memory is allocated here.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include "../../include/engram.h"
#include "launch.h"

using namespace engram;

namespace {

constexpr uint32_t kSpinBudget = 1u << 22;  // ~1 s of sleeping polls before a wait gives up

// From this many tokens on, the tiled schedule (256 x 256 MFMA tiles, each weight panel read
// once per 256 tokens) replaces weight streaming (all of wkv read once per 64 tokens).
constexpr int64_t kTiledMinTokens = 256;

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
  return M >= kTiledMinTokens &&
         tiled_shape_ok(int(N_of(l)), int(K_of(l)), l->dim, l->head_dim, l->scale_block, fused);
}

size_t forward_workspace(const engram_layout* l, int64_t M, int cus) {
  if (use_tiled(l, M, true)) return tiled_workspace_bytes(M, l->dim);
  return stream_workspace_bytes(M, int(N_of(l)), stream_grid(int(N_of(l)), cus));
}

}  // namespace

extern "C" {

const char* engram_status_str(engram_status s) {
  switch (s) {
    case ENGRAM_OK: return "ok";
    case ENGRAM_E_NULL: return "a required pointer is NULL";
    case ENGRAM_E_LAYOUT: return "invalid layout";
    case ENGRAM_E_SHAPE: return "invalid token count";
    case ENGRAM_E_ALIGN: return "tensor pointer not 16-byte aligned";
    case ENGRAM_E_WORKSPACE: return "workspace missing or too small";
    case ENGRAM_E_HIP: return "HIP runtime error";
    case ENGRAM_E_DEVICE: return "current device is not gfx950";
  }
  return "unknown status";
}

engram_status engram_layout_check(const engram_layout* l) {
  if (l == nullptr) return ENGRAM_E_NULL;
  if (l->hc != 4) return ENGRAM_E_LAYOUT;
  if (l->dim <= 0 || l->dim % 64 != 0) return ENGRAM_E_LAYOUT;
  if (l->n_cols <= 0 || l->head_dim <= 0 || l->head_dim % 64 != 0) return ENGRAM_E_LAYOUT;
  if (l->scale_block <= 0 || l->scale_block % 16 != 0 || l->head_dim % l->scale_block != 0)
    return ENGRAM_E_LAYOUT;
  if ((int64_t(l->n_cols) * l->head_dim) % 128 != 0) return ENGRAM_E_LAYOUT;
  if (int64_t(l->n_cols) * l->head_dim > (int64_t(1) << 20)) return ENGRAM_E_LAYOUT;
  if (l->reserved != 0 || l->n_rows <= 0) return ENGRAM_E_LAYOUT;
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

engram_status engram_gather_dequant(const engram_layout* l, const uint8_t* table, const float* scales,
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
  GatherArgs a{table, scales, hash_ids, M * l->n_cols, l->head_dim, l->scale_block, l->n_rows, emb, err_count};
  return launch_gather_dequant(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? ENGRAM_OK
                                                                                        : ENGRAM_E_HIP;
}

engram_status engram_kv_proj(const engram_layout* l, const uint16_t* emb, const uint16_t* wkv, int64_t B,
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
  if (use_tiled(l, M, false)) {
    TiledArgs a;
    memset(&a, 0, sizeof(a));
    a.wkv = wkv;
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
  a.wkv = wkv;
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
                             const uint8_t* token_mask, const uint8_t* table, const float* scales,
                             const uint16_t* wkv, const float* q_weight, const float* k_weight, int64_t B,
                             int64_t T, uint16_t* out, void* workspace, size_t workspace_bytes,
                             int32_t* err_count, engram_stream_t stream) {
  engram_status st = engram_layout_check(l);
  if (st != ENGRAM_OK) return st;
  int64_t M = 0;
  if ((st = check_tokens(B, T, &M)) != ENGRAM_OK) return st;
  if (M == 0) return ENGRAM_OK;
  if (!x || !hash_ids || !table || !scales || !wkv || !q_weight || !k_weight || !out) return ENGRAM_E_NULL;
  if (!aligned16(x) || !aligned16(table) || !aligned16(wkv) || !aligned16(q_weight) || !aligned16(k_weight) ||
      !aligned16(out) || (reinterpret_cast<uintptr_t>(scales) & 3u) || (reinterpret_cast<uintptr_t>(hash_ids) & 7u))
    return ENGRAM_E_ALIGN;
  DeviceInfo di;
  if ((st = device_info(&di)) != ENGRAM_OK) return st;
  const int N = int(N_of(l));
  const size_t need = forward_workspace(l, M, di.cus);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return ENGRAM_E_WORKSPACE;
  if (use_tiled(l, M, true)) {
    TiledArgs a;
    memset(&a, 0, sizeof(a));
    a.wkv = wkv;
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
    a.n_rows = l->n_rows;
    a.eps = l->eps;
    a.clamp = l->clamp;
    a.inv_sqrt_dim = float(1.0 / sqrt(double(l->dim)));
    a.spin_budget = kSpinBudget;
    return launch_forward_tiled(a, workspace, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? ENGRAM_OK
               : ENGRAM_E_HIP;
  }
  const int G = stream_grid(N, di.cus);
  if ((N / 16 + G - 1) / G > l->dim / 16) return ENGRAM_E_LAYOUT;
  StreamArgs a;
  memset(&a, 0, sizeof(a));
  a.wkv = wkv;
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
  a.n_rows = l->n_rows;
  a.eps = l->eps;
  a.clamp = l->clamp;
  a.inv_sqrt_dim = float(1.0 / sqrt(double(l->dim)));
  a.spin_budget = kSpinBudget;
  return launch_forward_stream(a, workspace, di.cus, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? ENGRAM_OK
             : ENGRAM_E_HIP;
}

}  // extern "C"
