// Internal definitions shared by the host and device halves of liblazyattn.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lazyattn.h"

namespace lazyattn {

constexpr int kBlock = 16;        // tokens per pool block
constexpr int kMaxPairs = 64;     // head_dim <= 128


// RoPE frequencies as revolutions per position: rev_i = theta^(-2i/D) / (2 pi),
// computed in double on the host.  Angles are reduced in double on the device
// (n * rev_i, fractional part) so that positions of tens of thousands keep
// ~1e-7 rad accuracy before the float sin/cos.
struct RopeRev {
  double rev[kMaxPairs];
};

// Table word: logical start in bits 63..32, physical block id in bits 31..0.
__host__ __device__ __forceinline__ uint64_t word_pack(uint32_t block, uint32_t start) {
  return (static_cast<uint64_t>(start) << 32) | static_cast<uint64_t>(block);
}
__host__ __device__ __forceinline__ uint32_t word_block(uint64_t w) {
  return static_cast<uint32_t>(w & 0xffffffffull);
}
__host__ __device__ __forceinline__ uint32_t word_start(uint64_t w) {
  return static_cast<uint32_t>(w >> 32);
}

// Host-side parameter checks shared by the entry points (lazyattn_host.cpp).
lazyattn_status check_config(const lazyattn_config* cfg);
RopeRev make_rope_rev(const lazyattn_config* cfg);
float softmax_scale_of(const lazyattn_config* cfg);

// Split heuristics and workspace sizes (host).
int prefill_rows_per_tile();  // query rows (positions x heads of one KV group) per work-group
int prefill_positions_per_tile(int group);
int choose_prefill_splits(const lazyattn_config* cfg, int num_reqs, int max_q_len, int max_entries);
int choose_decode_splits(const lazyattn_config* cfg, int num_reqs, int max_entries);
int prefill_entries_per_split(int max_entries, int splits);
// The prefill's key-turning route (LAZYATTN_FLAG_KEYS_ONCE) and its workspace:
// split partials first, then the turned keys from a 256-byte boundary
bool prefill_keys_once(const lazyattn_config* cfg, int max_q_len);
size_t prefill_partials_bytes(const lazyattn_config* cfg, int total_q, int splits);
size_t prefill_turned_keys_offset(size_t partials_bytes);
size_t prefill_turned_keys_bytes(const lazyattn_config* cfg, int num_reqs, int max_entries);
int decode_entries_per_split(int max_entries, int splits);
// decode work per (request, KV head, split) in 16-head work-groups: 2 for groups
// of more than 16 heads
int decode_halves(int group);

}  // namespace lazyattn
