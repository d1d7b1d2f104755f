// Host-only half of the C ABI: codec, table validation, split heuristics and
// workspace sizing.  Nothing here touches a GPU, so these entry points work
// on machines without one.
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "lazyattn_common.hpp"

namespace lazyattn {

lazyattn_status check_config(const lazyattn_config* cfg) {
  if (!cfg) return LAZYATTN_EINVAL;
  if (cfg->num_q_heads < 1 || cfg->num_kv_heads < 1) return LAZYATTN_EINVAL;
  if (cfg->num_q_heads % cfg->num_kv_heads != 0) return LAZYATTN_EINVAL;
  constexpr int32_t known = LAZYATTN_FLAG_EXACT_MAX | LAZYATTN_FLAG_KEYS_FUSED | LAZYATTN_FLAG_KEYS_ONCE;
  if ((cfg->flags & ~known) != 0) return LAZYATTN_EINVAL;
  if ((cfg->flags & LAZYATTN_FLAG_KEYS_FUSED) && (cfg->flags & LAZYATTN_FLAG_KEYS_ONCE)) return LAZYATTN_EINVAL;
  if (cfg->dtype != LAZYATTN_F32 && cfg->dtype != LAZYATTN_BF16) return LAZYATTN_EINVAL;
  if (cfg->pe != LAZYATTN_PE_ROPE && cfg->pe != LAZYATTN_PE_NONE && cfg->pe != LAZYATTN_PE_ALIBI)
    return LAZYATTN_EINVAL;
  if (cfg->pe == LAZYATTN_PE_ROPE && !cfg->rope_inv_freq && !(cfg->rope_theta > 0.0)) return LAZYATTN_EINVAL;
  if (!(cfg->softmax_scale >= 0.0f) || isinf(cfg->softmax_scale)) return LAZYATTN_EINVAL;
  if (cfg->head_dim < 1 || cfg->block_size < 1) return LAZYATTN_EINVAL;
  if (cfg->block_size != kBlock) return LAZYATTN_EUNSUPPORTED;
  if (cfg->dtype == LAZYATTN_BF16 && cfg->head_dim != 128) return LAZYATTN_EUNSUPPORTED;
  if (cfg->dtype == LAZYATTN_F32 && cfg->head_dim != 64 && cfg->head_dim != 128)
    return LAZYATTN_EUNSUPPORTED;
  if (cfg->kv_format != LAZYATTN_KV_PLAIN && cfg->kv_format != LAZYATTN_KV_FP8_E4M3) return LAZYATTN_EINVAL;
  if (cfg->kv_format == LAZYATTN_KV_FP8_E4M3 && (cfg->dtype != LAZYATTN_BF16 || cfg->head_dim != 128))
    return LAZYATTN_EUNSUPPORTED;
  if (cfg->rope_inv_freq) {
    for (int i = 0; i < cfg->head_dim / 2; ++i) {
      const double f = cfg->rope_inv_freq[i];
      if (!(f >= 0.0) || isinf(f)) return LAZYATTN_EINVAL;
    }
  }
  return LAZYATTN_OK;
}

RopeRev make_rope_rev(const lazyattn_config* cfg) {
  RopeRev r{};
  const int pairs = cfg->head_dim / 2;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < pairs && i < kMaxPairs; ++i) {
    const double inv_freq = cfg->rope_inv_freq
                                ? cfg->rope_inv_freq[i]
                                : pow(cfg->rope_theta > 0.0 ? cfg->rope_theta : 1.0,
                                      -2.0 * static_cast<double>(i) / static_cast<double>(cfg->head_dim));
    r.rev[i] = inv_freq / two_pi;
  }
  return r;
}

float softmax_scale_of(const lazyattn_config* cfg) {
  if (cfg->softmax_scale > 0.0f) return cfg->softmax_scale;
  return static_cast<float>(1.0 / sqrt(static_cast<double>(cfg->head_dim)));
}

// A prefill work-group holds 256 query rows: the G heads of one KV group at
// floor(256 / G) consecutive positions (position-major).
int prefill_rows_per_tile() { return 256; }
int prefill_positions_per_tile(int group) { return std::max(1, 256 / std::max(1, group)); }

static int ceil_div(long long a, long long b) { return static_cast<int>((a + b - 1) / b); }

int choose_prefill_splits(const lazyattn_config* cfg, int num_reqs, int max_q_len, int max_entries) {
  if (cfg->dtype != LAZYATTN_BF16) return 1;
  const int group = cfg->num_q_heads / cfg->num_kv_heads;
  const long long tiles = static_cast<long long>(ceil_div(std::max(1, max_q_len), prefill_positions_per_tile(group))) *
                          num_reqs * cfg->num_kv_heads;
  const int target = 256;  // one 8-wave work-group per compute unit
  if (tiles >= target) return 1;
  int s = ceil_div(target, std::max(1LL, tiles));
  // keep at least 16 key tiles (64 entries) per split
  s = std::min(s, std::max(1, max_entries / 64));
  return std::max(1, std::min(s, 64));
}

// The bf16 prefill over a plain content-only pool turns every key once before
// attending when asked to, or by default when a request spans at least
// LAZYATTN_KEYS_ONCE_TILES query tiles: each key is then staged by that many
// work-groups, and turning it in each of them costs more vector work than one
// pass that reads and writes the keys once.
bool prefill_keys_once(const lazyattn_config* cfg, int max_q_len) {
  if (cfg->dtype != LAZYATTN_BF16 || cfg->pe != LAZYATTN_PE_ROPE || cfg->kv_format != LAZYATTN_KV_PLAIN) return false;
  if (cfg->flags & LAZYATTN_FLAG_KEYS_FUSED) return false;
  if (cfg->flags & LAZYATTN_FLAG_KEYS_ONCE) return true;
  const int group = cfg->num_q_heads / cfg->num_kv_heads;
  return ceil_div(std::max(1, max_q_len), prefill_positions_per_tile(group)) >= LAZYATTN_KEYS_ONCE_TILES;
}

size_t prefill_partials_bytes(const lazyattn_config* cfg, int total_q, int splits) {
  if (splits <= 1) return 0;
  const size_t rows = static_cast<size_t>(total_q) * cfg->num_q_heads;
  return static_cast<size_t>(splits) * rows * (static_cast<size_t>(cfg->head_dim) * sizeof(uint16_t) + 2 * sizeof(float));
}

size_t prefill_turned_keys_offset(size_t partials_bytes) { return (partials_bytes + 255) / 256 * 256; }

size_t prefill_turned_keys_bytes(const lazyattn_config* cfg, int num_reqs, int max_entries) {
  return static_cast<size_t>(num_reqs) * static_cast<size_t>(std::max(0, max_entries)) * cfg->num_kv_heads * kBlock *
         cfg->head_dim * sizeof(uint16_t);
}

// Decode work per (request, KV head, split) in units of one 16-head work-group:
// groups of 17..32 heads take two (two work-groups of 16 heads, or one whose
// waves hold 32 columns and do twice the work per entry)
int decode_halves(int group) { return group > 16 ? 2 : 1; }

int choose_decode_splits(const lazyattn_config* cfg, int num_reqs, int max_entries) {
  if (cfg->dtype != LAZYATTN_BF16) return 1;
  const long long units = static_cast<long long>(num_reqs) * cfg->num_kv_heads *
                          decode_halves(cfg->num_q_heads / cfg->num_kv_heads);
  const int target = 512;   // two work-groups per compute unit: what the LDS reservation lets run at once
  if (units >= target) return 1;
  // one round of work-groups; when the longest request would then give a
  // split more than ~160 entries (the tail of a batch with mixed context
  // lengths), whole rounds more (a round and a bit would run a short second
  // round as long as the first; splits past a request's end exit at once)
  const int s0 = ceil_div(target, std::max(1LL, units));
  const int s1 = ceil_div(max_entries, 160);
  int s = s1 > s0 ? s0 * ceil_div(s1, s0) : s0;
  // keep at least 32 entries (8 per wave) per split
  s = std::min(s, std::max(1, max_entries / 32));
  return std::max(1, std::min(s, 256));
}

int prefill_entries_per_split(int max_entries, int splits) {
  int e = ceil_div(std::max(1, max_entries), std::max(1, splits));
  return (e + 3) / 4 * 4;  // whole 4-entry key tiles
}

int decode_entries_per_split(int max_entries, int splits) {
  return ceil_div(std::max(1, max_entries), std::max(1, splits));
}

}  // namespace lazyattn

using namespace lazyattn;

extern "C" {

int32_t lazyattn_abi_version(void) { return LAZYATTN_ABI_VERSION; }

lazyattn_status lazyattn_rope_inv_freq(int32_t head_dim, int32_t rotary_dim, double theta, double* out) {
  if (!out || head_dim < 2 || head_dim % 2 != 0 || rotary_dim < 2 || rotary_dim % 2 != 0 || rotary_dim > head_dim ||
      !(theta > 0.0) || isinf(theta))
    return LAZYATTN_EINVAL;
  for (int i = 0; i < head_dim / 2; ++i)
    out[i] = (2 * i < rotary_dim) ? pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(rotary_dim)) : 0.0;
  return LAZYATTN_OK;
}

lazyattn_status lazyattn_rope_inv_freq_llama31(int32_t head_dim, double theta, double factor, double low_freq_factor,
                                               double high_freq_factor, int32_t original_max_position, double* out) {
  if (!out || head_dim < 2 || head_dim % 2 != 0 || !(theta > 0.0) || isinf(theta) || !(factor >= 1.0) ||
      isinf(factor) || !(low_freq_factor > 0.0) || !(high_freq_factor > low_freq_factor) ||
      isinf(high_freq_factor) || original_max_position < 1)
    return LAZYATTN_EINVAL;
  const double two_pi = 6.283185307179586476925286766559;
  const double ctx = static_cast<double>(original_max_position);
  for (int i = 0; i < head_dim / 2; ++i) {
    const double f = pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(head_dim));
    const double wavelength = two_pi / f;
    if (wavelength < ctx / high_freq_factor) {
      out[i] = f;                                  // short wavelengths: unchanged
    } else if (wavelength > ctx / low_freq_factor) {
      out[i] = f / factor;                         // long wavelengths: stretched by the factor
    } else {
      const double s = (ctx / wavelength - low_freq_factor) / (high_freq_factor - low_freq_factor);
      out[i] = (1.0 - s) * (f / factor) + s * f;
    }
  }
  return LAZYATTN_OK;
}

const char* lazyattn_status_string(lazyattn_status s) {
  // callers may pass any integer: read it as one (an out-of-range value held in
  // the enum type must not be loaded as that type)
  int32_t v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case LAZYATTN_OK: return "ok";
    case LAZYATTN_EINVAL: return "invalid argument";
    case LAZYATTN_EUNSUPPORTED: return "unsupported configuration";
    case LAZYATTN_EWORKSPACE: return "workspace too small";
    case LAZYATTN_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

uint64_t lazyattn_pack(uint32_t block_id, uint32_t logical_start) {
  return word_pack(block_id, logical_start);
}
uint32_t lazyattn_entry_block(uint64_t word) { return word_block(word); }
uint32_t lazyattn_entry_start(uint64_t word) { return word_start(word); }

lazyattn_status lazyattn_pack_entries(const uint32_t* blocks, const uint32_t* starts, int64_t n,
                                      uint64_t* words) {
  if (n < 0) return LAZYATTN_EINVAL;
  if (n > 0 && (!blocks || !starts || !words)) return LAZYATTN_EINVAL;
  for (int64_t i = 0; i < n; ++i) words[i] = word_pack(blocks[i], starts[i]);
  return LAZYATTN_OK;
}

lazyattn_status lazyattn_validate_tables(const lazyattn_config* cfg, const uint64_t* tables_h,
                                         int32_t num_reqs, int32_t max_entries,
                                         const int32_t* num_entries_h, const int32_t* ctx_lens_h,
                                         int64_t num_blocks, int32_t* bad_req, int32_t* bad_entry) {
  if (bad_req) *bad_req = -1;
  if (bad_entry) *bad_entry = -1;
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if (num_reqs < 0 || max_entries < 0 || num_blocks < 0) return LAZYATTN_EINVAL;
  if (num_reqs > 0 && (!tables_h || !num_entries_h || !ctx_lens_h)) return LAZYATTN_EINVAL;
  const int64_t B = cfg->block_size;
  for (int32_t r = 0; r < num_reqs; ++r) {
    const int32_t n = num_entries_h[r];
    const int64_t L = ctx_lens_h[r];
    auto fail = [&](int32_t e) {
      if (bad_req) *bad_req = r;
      if (bad_entry) *bad_entry = e;
      return LAZYATTN_EINVAL;
    };
    if (n < 0 || n > max_entries || L < 0 || L > 0xffffffffLL) return fail(-1);
    if (n == 0) {
      if (L != 0) return fail(-1);
      continue;
    }
    const uint64_t* row = tables_h + static_cast<int64_t>(r) * max_entries;
    if (word_start(row[0]) != 0) return fail(0);
    for (int32_t e = 0; e < n; ++e) {
      const int64_t s = word_start(row[e]);
      const int64_t end = (e + 1 < n) ? static_cast<int64_t>(word_start(row[e + 1])) : L;
      const int64_t len = end - s;
      if (len < 1 || len > B) return fail(e);
      if (static_cast<int64_t>(word_block(row[e])) >= num_blocks) return fail(e);
    }
  }
  return LAZYATTN_OK;
}

int32_t lazyattn_prefill_splits(const lazyattn_config* cfg, int32_t num_reqs, int32_t max_q_len,
                                int32_t max_entries) {
  if (check_config(cfg) != LAZYATTN_OK) return 0;
  return choose_prefill_splits(cfg, num_reqs, max_q_len, max_entries);
}

int32_t lazyattn_prefill_splits_balanced(const lazyattn_config* cfg, int32_t num_reqs, int32_t max_q_len,
                                         int32_t max_entries, int64_t total_entries) {
  if (check_config(cfg) != LAZYATTN_OK) return 0;
  int s = choose_prefill_splits(cfg, num_reqs, max_q_len, max_entries);
  if (num_reqs < 1 || total_entries < 1 || max_entries < 1 || cfg->dtype != LAZYATTN_BF16) return s;
  // ceil(longest / mean - 0.1): the longest request's share per work-group comes down to about
  // the mean's (a ratio within 0.1 above a whole number does not take one more split)
  const long long num = 10LL * max_entries * num_reqs - total_entries, den = 10LL * total_entries;
  const long long imb = std::max(1LL, (num + den - 1) / den);
  const long long cap = std::max(1, max_entries / 64);   // at least 16 key tiles per split
  const long long want = std::min<long long>(imb, cap);
  return static_cast<int32_t>(std::max<long long>(s, std::min<long long>(want, 64)));
}

int32_t lazyattn_decode_splits(const lazyattn_config* cfg, int32_t num_reqs, int32_t max_entries) {
  if (check_config(cfg) != LAZYATTN_OK) return 0;
  return choose_decode_splits(cfg, num_reqs, max_entries);
}

size_t lazyattn_prefill_workspace_size(const lazyattn_config* cfg, int32_t num_reqs, int32_t total_q,
                                       int32_t max_q_len, int32_t max_entries, int32_t num_splits) {
  if (check_config(cfg) != LAZYATTN_OK || num_reqs < 0 || total_q < 0) return 0;
  if (cfg->dtype != LAZYATTN_BF16) return 0;  // the fp32 path never splits
  int s = num_splits > 0 ? num_splits : choose_prefill_splits(cfg, num_reqs, max_q_len, max_entries);
  const size_t part = prefill_partials_bytes(cfg, total_q, s);
  if (!prefill_keys_once(cfg, max_q_len) || num_reqs == 0) return part;
  return prefill_turned_keys_offset(part) + prefill_turned_keys_bytes(cfg, num_reqs, max_entries);
}

size_t lazyattn_decode_workspace_size(const lazyattn_config* cfg, int32_t num_reqs,
                                      int32_t max_entries, int32_t num_splits) {
  if (check_config(cfg) != LAZYATTN_OK || num_reqs < 0) return 0;
  if (cfg->dtype != LAZYATTN_BF16) return 0;  // the fp32 path never splits
  int s = num_splits > 0 ? num_splits : choose_decode_splits(cfg, num_reqs, max_entries);
  if (s <= 1) return 0;
  const size_t rows = static_cast<size_t>(num_reqs) * cfg->num_q_heads;
  return static_cast<size_t>(s) * rows * (static_cast<size_t>(cfg->head_dim) * sizeof(uint16_t) + 2 * sizeof(float));
}

}  // extern "C"
