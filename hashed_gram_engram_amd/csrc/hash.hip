// The hash step in front of the Engram path: raw token ids -> the global row ids of every
// Engram layer (engram-second page, code panel, the hash module's forward; "DeepSeek's Other
// Modules", Engram, The lookup pipeline).
//
// One thread per token.  Look-back `shift` of position p reads the compressed id of position
// p - shift: inside this call from the token map directly (so no thread waits for another's
// history write), before it from the caller's history; a look-back before the sequence start or
// onto a dead token, and every longer look-back after it, reads pad_id.  For every layer the
// products token x multiplier wrap modulo 2^64 (two's complement, as int64 tensors do), their
// running XOR over look-backs 0..i is the (i+1)-gram's hash, and head k's row id is that value
// modulo the head's prime (floor modulo: in [0, p)) plus the column's offset.  Each thread
// also stores its own compressed id into the history for later calls.
#include "common.h"
#include "launch.h"

namespace engram {

namespace {

constexpr int kMaxNgram = 8;

__global__ __launch_bounds__(256) void k_hash_ids(HashArgs a) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= a.B * a.L) return;
  const int64_t b = i / a.L, l = i - b * a.L;
  const int64_t pos = a.start_pos + l;
  // compressed id of a token of this call (dead: masked, or an id outside the map)
  auto compressed = [&](int64_t ll) -> int64_t {
    const int64_t id = a.input_ids[b * a.L + ll];
    if (id < 0 || id >= a.vocab) return kDead;
    if (a.token_mask != nullptr && a.token_mask[b * a.L + ll] == 0) return kDead;
    return int64_t(a.token_map[id]);
  };
  {
    const int64_t id = a.input_ids[i];
    if ((id < 0 || id >= a.vocab) && a.err_count != nullptr) atomicAdd(a.err_count, 1);
  }
  uint64_t tok[kMaxNgram];
  bool blocked = false;
  for (int sh = 0; sh < a.max_ngram; ++sh) {
    int64_t src = kDead;
    if (pos - sh >= 0) src = l - sh >= 0 ? compressed(l - sh) : a.history[b * a.history_len + pos - sh];
    blocked = blocked || pos < sh || src == kDead;
    tok[sh] = uint64_t(blocked ? int64_t(a.pad_id) : src);
  }
  a.history[b * a.history_len + pos] = compressed(l);
  const int n_cols = (a.max_ngram - 1) * a.n_heads;
  for (int layer = 0; layer < a.n_layers; ++layer) {
    const int64_t* mult = a.multipliers + layer * a.max_ngram;
    int64_t* out = a.hash_ids + ((int64_t(layer) * a.B + b) * a.L + l) * n_cols;
    uint64_t rolling = tok[0] * uint64_t(mult[0]);
    for (int n = 1; n < a.max_ngram; ++n) {
      rolling ^= tok[n] * uint64_t(mult[n]);
      const int64_t h = int64_t(rolling);
      for (int k = 0; k < a.n_heads; ++k) {
        const int col = (n - 1) * a.n_heads + k;
        const int64_t p = a.primes[(int64_t(layer) * (a.max_ngram - 1) + (n - 1)) * a.n_heads + k];
        int64_t r = -1;
        if (p > 0) {
          r = h % p;
          r = r < 0 ? r + p : r;
          r += a.offsets[int64_t(layer) * n_cols + col];
        } else if (a.err_count != nullptr) {
          atomicAdd(a.err_count, 1);
        }
        out[col] = r;
      }
    }
  }
}

}  // namespace

hipError_t launch_hash_ids(const HashArgs& a, hipStream_t stream) {
  const int64_t n = a.B * a.L;
  if (n <= 0) return hipSuccess;
  if (a.max_ngram < 2 || a.max_ngram > kMaxNgram) return hipErrorInvalidValue;
  const int64_t grid = (n + 255) / 256;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  HashArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&k_hash_ids), dim3(unsigned(grid)), dim3(256), params, 0,
                         stream);
}

}  // namespace engram
