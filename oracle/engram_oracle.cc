// CPU oracle of the DeepSeek-V4.1-Flash Engram forward.  TEST INFRASTRUCTURE ONLY.
//
// Only the tests, __graft_entry__.smoke() and the cpu_baseline leg of bench.py load this
// library (through oracle/__init__.py).  The product library (libengram.so) never links it, and
// the two share no source, header, helper or constant table.
//
// What it computes is the plain definition of the Engram block, written from the pages:
//  * "DeepSeek-V4.1 / blocks / engram-second" (atlas.klimoza.dev), code panel: Engram.forward and
//    ParallelEngramEmbedding.forward (gather fp8 rows and their block scales, multiply in fp32,
//    round to bf16, flatten the hash columns, project with wkv into four keys and one value,
//    gate each stream by a normalised dot product, add gate x value to every stream).
//  * "DeepSeek's Other Modules" (monishver11.github.io), section Engram: The lookup pipeline
//    (compressed ids, one odd multiplier per look-back, XOR, modulo a prime per head; shared
//    value, one key and gate per stream), V4.1's two tables, reconciled (24 columns of 256 fp8
//    features, the 6,144 -> 25,600 projection).
//  * "Engram in DeepSeek V4.1 Flash" (zhuai.tech): Step 1 (token -> compressed id -> the current
//    and three preceding positions -> 24 hashes -> 24 row addresses), Step 3 (the gate restated,
//    per stream, q and k used as their product), Step 4 (one history per session; image spans
//    insert dead markers that n-grams do not cross).
//
// Precision: every floating-point step is carried out in IEEE double, except where the pages fix
// a narrower type, which is then applied as an explicit rounding:
//  * the dequantisation product is an fp32 multiply (fp8 value times its block scale);
//  * table rows are rounded to bf16 before the projection;
//  * the projection output kv is rounded to bf16 through fp32 (the Linear keeps the bf16
//    activation dtype; the sum of exact bf16 x bf16 products is taken in double, in feature
//    order, then rounded once to fp32 and once to bf16);
//  * q_weight * k_weight is an fp32 product;
//  * the output streams are rounded to bf16 through fp32.
// Reductions start from +0, so an all-zero sum is +0.  Every result of a token depends on that
// token alone, so work is spread over threads by token; the result does not depend on the
// number of threads.
//
// Plain C++17, built with g++ -O2 -ffp-contract=off (no fused multiply-add, no reassociation).

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ------------------------------------------------------------------------------------------
// number formats
// ------------------------------------------------------------------------------------------

// OCP FP8 E4M3 "fn" (torch.float8_e4m3fn, the table dtype of ParallelEngramEmbedding on the
// engram-second page): sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities.
// Exponent field 15 with mantissa 7 is NaN; exponent field 0 is subnormal, m * 2^-9.
double e4m3_value(uint8_t code) {
  const int sign = code >> 7;
  const int e = (code >> 3) & 15;
  const int m = code & 7;
  if (e == 15 && m == 7) return std::nan("");
  const double mag = (e == 0) ? std::ldexp(double(m), -9) : std::ldexp(double(8 + m), e - 10);
  return sign ? -mag : mag;
}

// OCP Microscaling v1.0 scale E8M0 (the block scale of the MXFP8 tables, "Engram in DeepSeek
// V4.1 Flash", Step 2): an unsigned biased exponent, 2^(e - 127), e = 255 is NaN.
double e8m0_value(uint8_t e) {
  if (e == 255) return std::nan("");
  return std::ldexp(1.0, int(e) - 127);
}

// Nearest fp32 (ties to even) of a double, as a double.  The conversion is the IEEE one of the
// host (round to nearest even; out of range gives an infinity).
double to_fp32(double v) { return double(static_cast<float>(v)); }

// bf16 bit pattern of a value that is already an fp32 number: round the low 16 bits away,
// nearest with ties to even; NaN becomes the canonical quiet NaN 0x7FC0.
uint16_t bf16_of_fp32(float f) {
  if (std::isnan(f)) return 0x7FC0;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  const uint32_t low = u & 0xFFFFu;
  uint32_t top = u >> 16;
  if (low > 0x8000u || (low == 0x8000u && (top & 1u))) top += 1;  // may carry into the exponent
  return uint16_t(top);
}

// bf16 of a double, through fp32 (both roundings to nearest even).
uint16_t bf16_of(double v) { return bf16_of_fp32(static_cast<float>(v)); }

double bf16_value(uint16_t bits) {
  const uint32_t u = uint32_t(bits) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return double(f);
}

// ------------------------------------------------------------------------------------------
// threads over tokens
// ------------------------------------------------------------------------------------------

template <class F>
void for_each_token(int64_t M, int threads, F&& body) {
  if (threads < 1) threads = int(std::thread::hardware_concurrency());
  if (threads < 1) threads = 1;
  if (int64_t(threads) > M) threads = int(M > 0 ? M : 1);
  if (threads == 1) {
    for (int64_t m = 0; m < M; ++m) body(m);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> pool;
  pool.reserve(threads);
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([&] {
      for (int64_t m = next++; m < M; m = next++) body(m);
    });
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// ------------------------------------------------------------------------------------------
// number formats, element-wise
// ------------------------------------------------------------------------------------------

void orc_e4m3_values(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(codes[i]);
}

void orc_e8m0_values(const uint8_t* e, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e8m0_value(e[i]);
}

void orc_round_fp32(const double* x, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = to_fp32(x[i]);
}

void orc_bf16_from_double(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_of(x[i]);
}

void orc_bf16_values(const uint16_t* bits, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_value(bits[i]);
}

// ------------------------------------------------------------------------------------------
// S1 + S2: row gather and dequantisation
// ------------------------------------------------------------------------------------------

// The table as the oracle holds it: either every row (row_ids == NULL: row r is held at
// position r), or a subset of rows named by the ascending row_ids[0 .. n_held), each held at its
// position in that list (a host cannot hold a 98 GB table; the rows a test's tokens touch are
// enough).  codes [n_held, head_dim] e4m3fn bytes; scales [n_held, head_dim / scale_block] fp32
// (scale_format 0) or E8M0 bytes (scale_format 1).
struct Rows {
  const uint8_t* codes;
  const void* scales;
  const int64_t* row_ids;
  int64_t n_held;
};

// Position of global row r in the held rows, or -1 if it is not held.
static int64_t held_position(const Rows& t, int64_t r) {
  if (t.row_ids == nullptr) return (r < t.n_held) ? r : -1;
  int64_t lo = 0, hi = t.n_held;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (t.row_ids[mid] < r) lo = mid + 1; else hi = mid;
  }
  return (lo < t.n_held && t.row_ids[lo] == r) ? lo : -1;
}

static double block_scale(const Rows& t, int64_t pos, int nb, int b, int scale_format) {
  if (scale_format == 1) return e8m0_value(static_cast<const uint8_t*>(t.scales)[pos * nb + b]);
  return double(static_cast<const float*>(t.scales)[pos * nb + b]);
}

// One token: emb[j * head_dim + c] for its C row ids (engram-second page,
// ParallelEngramEmbedding.forward with one shard, then Engram.forward's flatten).  A row id
// outside [0, n_rows) is a row this shard does not hold: it reads as zeros.  Returns -1 if an
// in-range row is missing from the held rows.
static int gather_token(const int64_t* ids, int C, int64_t n_rows, int head_dim, int scale_block,
                        int scale_format, const Rows& t, uint16_t* emb) {
  const int nb = head_dim / scale_block;
  for (int j = 0; j < C; ++j) {
    uint16_t* dst = emb + int64_t(j) * head_dim;
    const int64_t r = ids[j];
    if (r < 0 || r >= n_rows) {
      for (int c = 0; c < head_dim; ++c) dst[c] = 0;
      continue;
    }
    const int64_t pos = held_position(t, r);
    if (pos < 0) return -1;
    const uint8_t* row = t.codes + pos * head_dim;
    for (int c = 0; c < head_dim; ++c) {
      const double s = block_scale(t, pos, nb, c / scale_block, scale_format);
      // fp8 value times an fp32 scale: the exact product has at most 4 + 24 significant bits,
      // so the double product is exact and one rounding gives the IEEE fp32 product
      const double prod = to_fp32(e4m3_value(row[c]) * s);
      dst[c] = bf16_of(prod);
    }
  }
  return 0;
}

int orc_gather_dequant(const int64_t* hash_ids, int64_t M, int32_t C, int64_t n_rows,
                       int32_t head_dim, int32_t scale_block, int32_t scale_format,
                       const uint8_t* codes, const void* scales, const int64_t* row_ids,
                       int64_t n_held, uint16_t* emb, int32_t threads) {
  const Rows t{codes, scales, row_ids, n_held};
  std::atomic<int> bad{0};
  for_each_token(M, threads, [&](int64_t m) {
    if (gather_token(hash_ids + m * C, C, n_rows, head_dim, scale_block, scale_format, t,
                     emb + m * int64_t(C) * head_dim) != 0)
      bad = 1;
  });
  return bad ? -1 : 0;
}

// FP8 projection weights (a reading: "DeepSeek's Other Modules" says the projections are FP8
// like the tables without a scale layout; the tables' MXFP8 form along the input features):
// weight (n, k) = bf16(fp32(e4m3(codes[n, k]) * 2^(exps[n, k / 32] - 127))).
void orc_wkv_mxfp8_bits(const uint8_t* codes, const uint8_t* exps, int64_t N, int64_t K,
                        uint16_t* out) {
  const int64_t nb = K / 32;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      out[n * K + k] = bf16_of(to_fp32(e4m3_value(codes[n * K + k]) * e8m0_value(exps[n * nb + k / 32])));
}

// ------------------------------------------------------------------------------------------
// S3: the wkv projection
// ------------------------------------------------------------------------------------------

// Weight (n, k) as a double: bf16 bit patterns or fp32 values that are bf16 numbers.
struct Weights {
  const uint16_t* bf16;
  const float* f32;
  double at(int64_t i) const { return bf16 ? bf16_value(bf16[i]) : double(f32[i]); }
};

// kv[n] = bf16(fp32(sum_k emb[k] * wkv[n, k])) of one token (engram-second page,
// self.wkv = Linear(n_hash_cols * head_dim, dim * (hc_mult + 1)), weight [out, in]).  The
// product of two bf16 numbers is exact in double; the sum runs over k in order from +0.
static void project_token(const uint16_t* emb, const Weights& w, int64_t N, int64_t K,
                          uint16_t* kv, double* exact, std::vector<double>& a) {
  a.resize(K);
  for (int64_t k = 0; k < K; ++k) a[k] = bf16_value(emb[k]);
  for (int64_t n = 0; n < N; ++n) {
    double s = 0.0;
    const int64_t base = n * K;
    if (w.bf16) {
      for (int64_t k = 0; k < K; ++k) s += a[k] * bf16_value(w.bf16[base + k]);
    } else {
      for (int64_t k = 0; k < K; ++k) s += a[k] * double(w.f32[base + k]);
    }
    kv[n] = bf16_of(s);
    if (exact) exact[n] = s;
  }
}

void orc_kv_proj(const uint16_t* emb, const uint16_t* wkv_bf16, const float* wkv_f32, int64_t M,
                 int64_t N, int64_t K, uint16_t* kv, double* exact, int32_t threads) {
  const Weights w{wkv_bf16, wkv_f32};
  for_each_token(M, threads, [&](int64_t m) {
    std::vector<double> a;
    project_token(emb + m * K, w, N, K, kv + m * N, exact ? exact + m * N : nullptr, a);
  });
}

// ------------------------------------------------------------------------------------------
// S4 + S5: the per-(token, stream) gate; S6: the residual add
// ------------------------------------------------------------------------------------------

struct GateParts {
  double A, Kq, D, dot, gate;
};

// Gate of stream s of one token (engram-second page, Engram.forward; zhuai.tech Step 3): with
// h = x as double, key = the stream's dim columns of kv and w = fl32(q * k),
//   rstd = 1/sqrt(mean h^2 + eps) * 1/sqrt(mean key^2 + eps),
//   dot  = (sum_d h * w * key) * rstd * dim^-1/2,
//   gate = sigmoid(copysign(sqrt(max(|dot|, clamp)), dot)),
// normalised for each (token, stream) alone; 0 where the token's mask is false.
static GateParts gate_of(const uint16_t* x_s, const uint16_t* key, const float* q_s,
                         const float* k_s, int dim, double eps, double clamp, bool open) {
  GateParts p{0.0, 0.0, 0.0, 0.0, 0.0};
  for (int d = 0; d < dim; ++d) {
    const double h = bf16_value(x_s[d]);
    const double kk = bf16_value(key[d]);
    const double w = to_fp32(double(q_s[d]) * double(k_s[d]));  // exact double product, rounded
    p.A += h * h;
    p.Kq += kk * kk;
    p.D += (h * w) * kk;
  }
  const double rstd = (1.0 / std::sqrt(p.A / dim + eps)) * (1.0 / std::sqrt(p.Kq / dim + eps));
  p.dot = p.D * rstd * (1.0 / std::sqrt(double(dim)));
  const double z = std::copysign(std::sqrt(std::fmax(std::fabs(p.dot), clamp)), p.dot);
  p.gate = open ? 1.0 / (1.0 + std::exp(-z)) : 0.0;
  return p;
}

// out = h + gate * value for one stream of one token, the value shared by all streams
// (engram-second page, the last line of Engram.forward; zhuai.tech Step 3, hidden += gate x
// value).  A token whose mask is false passes through untouched (the Engram.forward docstring).
static void residual_stream(const uint16_t* x_s, const uint16_t* value, double g, int dim,
                            bool open, double* out_f, uint16_t* out_bits) {
  for (int d = 0; d < dim; ++d) {
    const double h = bf16_value(x_s[d]);
    const double o = open ? h + g * bf16_value(value[d]) : h;
    if (out_f) out_f[d] = o;
    if (out_bits) out_bits[d] = open ? bf16_of(o) : x_s[d];
  }
}

// S4 - S6 of one token from its kv; every output pointer may be NULL.
static void gate_apply_token(const uint16_t* x, const uint16_t* kv, const float* q,
                             const float* k, bool open, int hc, int dim, double eps, double clamp,
                             double* gate, double* A, double* Kq, double* D, double* dot,
                             double* out_f, uint16_t* out_bits) {
  const uint16_t* value = kv + int64_t(hc) * dim;
  for (int s = 0; s < hc; ++s) {
    const GateParts p = gate_of(x + int64_t(s) * dim, kv + int64_t(s) * dim, q + int64_t(s) * dim,
                                k + int64_t(s) * dim, dim, eps, clamp, open);
    if (gate) gate[s] = p.gate;
    if (A) A[s] = p.A;
    if (Kq) Kq[s] = p.Kq;
    if (D) D[s] = p.D;
    if (dot) dot[s] = p.dot;
    residual_stream(x + int64_t(s) * dim, value, p.gate, dim, open,
                    out_f ? out_f + int64_t(s) * dim : nullptr,
                    out_bits ? out_bits + int64_t(s) * dim : nullptr);
  }
}

// x [M, hc, dim] bf16, kv [M, (hc + 1) * dim] bf16, q/k [hc, dim] fp32, mask [M] (NULL: all
// open); outputs gate/A/Kq/D/dot [M, hc], out_f [M, hc, dim] double, out_bits [M, hc, dim] bf16,
// each NULL to skip.
void orc_gate_apply(const uint16_t* x, const uint16_t* kv, const float* q, const float* k,
                    const uint8_t* mask, int64_t M, int32_t hc, int32_t dim, double eps,
                    double clamp, double* gate, double* A, double* Kq, double* D, double* dot,
                    double* out_f, uint16_t* out_bits, int32_t threads) {
  const int64_t xs = int64_t(hc) * dim, kvs = int64_t(hc + 1) * dim;
  for_each_token(M, threads, [&](int64_t m) {
    const bool open = mask ? mask[m] != 0 : true;
    gate_apply_token(x + m * xs, kv + m * kvs, q, k, open, hc, dim, eps, clamp,
                     gate ? gate + m * hc : nullptr, A ? A + m * hc : nullptr,
                     Kq ? Kq + m * hc : nullptr, D ? D + m * hc : nullptr,
                     dot ? dot + m * hc : nullptr, out_f ? out_f + m * xs : nullptr,
                     out_bits ? out_bits + m * xs : nullptr);
  });
}

// S6 alone with a given gate [M, hc] (double).
void orc_residual(const uint16_t* x, const uint16_t* kv, const double* gate, const uint8_t* mask,
                  int64_t M, int32_t hc, int32_t dim, double* out_f, uint16_t* out_bits) {
  const int64_t xs = int64_t(hc) * dim, kvs = int64_t(hc + 1) * dim;
  for (int64_t m = 0; m < M; ++m) {
    const bool open = mask ? mask[m] != 0 : true;
    for (int s = 0; s < hc; ++s)
      residual_stream(x + m * xs + int64_t(s) * dim, kv + m * kvs + int64_t(hc) * dim,
                      gate[m * hc + s], dim, open, out_f ? out_f + m * xs + int64_t(s) * dim : nullptr,
                      out_bits ? out_bits + m * xs + int64_t(s) * dim : nullptr);
  }
}

// ------------------------------------------------------------------------------------------
// the whole forward
// ------------------------------------------------------------------------------------------

// Engram.forward for M tokens, each on its own: gather + dequantise its C rows, project, gate,
// add.  Outputs emb [M, C * head_dim], kv [M, N], gate [M, hc], out_f [M, hc, dim],
// out_bits [M, hc, dim]; each may be NULL.  Returns -1 if a needed row is not held.
int orc_forward(const uint16_t* x, const int64_t* hash_ids, const uint8_t* mask, int64_t M,
                int32_t hc, int32_t dim, int32_t C, int32_t head_dim, int32_t scale_block,
                int32_t scale_format, int64_t n_rows, const uint8_t* codes, const void* scales,
                const int64_t* row_ids, int64_t n_held, const uint16_t* wkv_bf16,
                const float* wkv_f32, const float* q, const float* k, double eps, double clamp,
                uint16_t* emb_out, uint16_t* kv_out, double* gate_out, double* out_f,
                uint16_t* out_bits, int32_t threads) {
  const Rows t{codes, scales, row_ids, n_held};
  const Weights w{wkv_bf16, wkv_f32};
  const int64_t K = int64_t(C) * head_dim, N = int64_t(hc + 1) * dim, xs = int64_t(hc) * dim;
  std::atomic<int> bad{0};
  for_each_token(M, threads, [&](int64_t m) {
    std::vector<uint16_t> emb(K), kv(N);
    std::vector<double> a;
    if (gather_token(hash_ids + m * C, C, n_rows, head_dim, scale_block, scale_format, t,
                     emb.data()) != 0) {
      bad = 1;
      return;
    }
    project_token(emb.data(), w, N, K, kv.data(), nullptr, a);
    const bool open = mask ? mask[m] != 0 : true;
    gate_apply_token(x + m * xs, kv.data(), q, k, open, hc, dim, eps, clamp,
                     gate_out ? gate_out + m * hc : nullptr, nullptr, nullptr, nullptr, nullptr,
                     out_f ? out_f + m * xs : nullptr, out_bits ? out_bits + m * xs : nullptr);
    if (emb_out) std::memcpy(emb_out + m * K, emb.data(), K * sizeof(uint16_t));
    if (kv_out) std::memcpy(kv_out + m * N, kv.data(), N * sizeof(uint16_t));
  });
  return bad ? -1 : 0;
}

// ------------------------------------------------------------------------------------------
// the hash step in front of the path: token ids -> the row ids of every Engram layer
// ------------------------------------------------------------------------------------------

// Row ids of the tokens input_ids [B, L] at positions start_pos .. start_pos + L - 1 of their
// sequences, for every Engram layer ("DeepSeek's Other Modules", Engram, The lookup pipeline;
// "Engram in DeepSeek V4.1 Flash", Step 1 and Step 4; shapes from the engram-second page):
//
//  1. A token's compressed id is token_map[id]; a token whose mask is false (an image span) is
//     the dead marker instead.  Each position's compressed id enters the sequence's history
//     once (history[b, p]); earlier positions come from earlier calls.
//  2. The n-gram ending at position p is read backwards: look-back s = 0, 1, ..., max_ngram - 1
//     is the compressed id at p - s.  From the first look-back that falls before the start of
//     the sequence or lands on a dead marker, that look-back and every longer one read pad_id,
//     so no n-gram reaches across a sequence start or an image.
//  3. For layer y, look-back s contributes its id times the layer's odd multiplier for s; the
//     contributions are combined by XOR.  After folding in look-backs 0..n (n >= 1) the value is
//     the hash of the (n+1)-gram; head k of that order takes it modulo its prime (the result
//     taken in [0, prime)), and the column's offset moves it into the column's row range.
//
// Output: out[b, l, y, (n - 1) * n_heads + k], int64.  Products: wide == 0 multiplies and XORs
// modulo 2^64 and reads the result as a two's-complement int64 (the model's int64 tensors);
// wide == 1 keeps them exact in 128 bits, ids and multipliers taken as non-negative (the
// Python-integer demo on "DeepSeek's Other Modules").  Returns the number of input ids outside
// [0, vocab) (those are treated as dead), or -1 on an invalid argument.
int64_t orc_hash_ids(const int64_t* input_ids, const uint8_t* token_mask, int64_t B, int64_t L,
                     const int64_t* token_map, int64_t vocab, const uint64_t* multipliers,
                     const int64_t* primes, const int64_t* offsets, int32_t n_layers,
                     int32_t max_ngram, int32_t n_heads, int64_t pad_id, int64_t dead,
                     int64_t* history, int64_t history_len, int64_t start_pos, int32_t wide,
                     int64_t* out) {
  if (max_ngram < 2 || max_ngram > 16 || n_layers < 1 || n_heads < 1 || start_pos < 0 ||
      start_pos + L > history_len)
    return -1;
  for (int64_t i = 0; i < int64_t(n_layers) * (max_ngram - 1) * n_heads; ++i)
    if (primes[i] <= 0) return -1;
  const int64_t n_cols = int64_t(max_ngram - 1) * n_heads;
  int64_t bad_ids = 0;
  // step 1: this call's positions enter the history
  for (int64_t b = 0; b < B; ++b)
    for (int64_t l = 0; l < L; ++l) {
      const int64_t id = input_ids[b * L + l];
      int64_t c = dead;
      if (id < 0 || id >= vocab) ++bad_ids;
      else if (token_mask == nullptr || token_mask[b * L + l] != 0) c = token_map[id];
      history[b * history_len + start_pos + l] = c;
    }
  for (int64_t b = 0; b < B; ++b)
    for (int64_t l = 0; l < L; ++l) {
      const int64_t p = start_pos + l;
      // step 2: the look-back window, padded from the first position it may not read
      int64_t window[16];
      bool readable = true;
      for (int s = 0; s < max_ngram; ++s) {
        const int64_t q = p - s;
        if (q < 0 || history[b * history_len + q] == dead) readable = false;
        window[s] = readable ? history[b * history_len + q] : pad_id;
      }
      // step 3: per layer, fold the look-backs in with XOR and reduce each order's hash
      for (int y = 0; y < n_layers; ++y) {
        int64_t* dst = out + ((b * L + l) * n_layers + y) * n_cols;
        const int64_t* pr = primes + int64_t(y) * (max_ngram - 1) * n_heads;
        const int64_t* off = offsets + int64_t(y) * n_cols;
        uint64_t h64 = 0;
        unsigned __int128 h128 = 0;
        for (int s = 0; s < max_ngram; ++s) {
          const uint64_t mult = multipliers[int64_t(y) * max_ngram + s];
          if (wide) h128 ^= (unsigned __int128)(uint64_t)window[s] * mult;
          else h64 ^= (uint64_t)window[s] * mult;  // unsigned arithmetic wraps modulo 2^64
          if (s == 0) continue;
          for (int k = 0; k < n_heads; ++k) {
            const int64_t prime = pr[(s - 1) * n_heads + k];
            int64_t r;
            if (wide) {
              r = int64_t(h128 % (unsigned __int128)prime);
            } else {
              const int64_t v = int64_t(h64);           // two's-complement reading
              r = v % prime;                            // C++ truncates toward zero ...
              if (r < 0) r += prime;                    // ... the hash takes [0, prime)
            }
            const int64_t col = int64_t(s - 1) * n_heads + k;
            dst[col] = r + off[col];
          }
        }
      }
    }
  return bad_ids;
}

// ------------------------------------------------------------------------------------------
// layout accounting
// ------------------------------------------------------------------------------------------

// Learned element counts of one Engram instance (engram-second page, Parameters table): table
// rows x features, the wkv projection, the q and k gate weights; out[3] is their sum.
void orc_param_counts(int64_t n_rows, int64_t head_dim, int64_t n_cols, int64_t hc, int64_t dim,
                      int64_t out[4]) {
  out[0] = n_rows * head_dim;
  out[1] = (n_cols * head_dim) * (dim * (hc + 1));
  out[2] = 2 * hc * dim;
  out[3] = out[0] + out[1] + out[2];
}

// Table traffic of one token in one module: one fp8 byte per feature of each gathered row and one
// scale per block ("DeepSeek's Other Modules", Serving cost).  out = {code bytes, scale bytes}.
void orc_bytes_per_token(int64_t n_cols, int64_t head_dim, int64_t scale_block, int64_t scale_bytes,
                         int64_t out[2]) {
  out[0] = n_cols * head_dim;
  out[1] = n_cols * (head_dim / scale_block) * scale_bytes;
}

}  // extern "C"
