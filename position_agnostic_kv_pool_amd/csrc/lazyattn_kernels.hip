// HIP kernels for gfx950 (CDNA4) and the GPU half of the C ABI.
//
// Method: LazyAttention ("LazyAttention: Efficient Retrieval-Augmented
// Generation with Deferred Positional Encoding").  The pool holds content-only
// keys (gist.science explainer, Technical Summary > Methodology > Core
// Concept); RoPE is applied inside the kernels at each request's logical
// positions.  Because R(a)^T R(b) = R(b - a), a query at p and a key at t
// score q^T R(t - p) k (gist.science, Mathematical Equivalence), so each
// kernel only needs relative rotations:
//  - prefill: the query tile is rotated once by R(m) (m = row offset within
//    the tile); every key of a key tile is rotated once by R(t - p0) (p0 =
//    tile base) while it is staged into LDS, and that rotated tile is shared
//    by every query row and every head of the KV group (gist.science,
//    Technical Implementation > Prefilling: one relative rotation per tile);
//    a chunk of many query tiles instead has every key of a request turned
//    once by R(t - c) (c = the request's first new position) in a pass of its
//    own (turn_keys_kernel), and the attention kernel turns only the queries,
//    by R(m - c);
//  - decode: each key row r of a block starting at S is rotated by
//    R(S - p + r) = R(S - p) R(r); R(S - p) is formed once per block and
//    R(r) is a per-lane constant (gist.science, Technical Implementation >
//    Decoding: the rotation is fused into the inner loop; only K and V are
//    read, the block metadata is one 64-bit word).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "lazyattn_common.hpp"

namespace lazyattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// e^{i n f} for the integer offset n, f = 2 pi rev: the angle is reduced to a
// fraction of a turn in double, then sin/cos are taken in float.
__device__ __forceinline__ float2 unit_phase(int n, double rev) {
  double x = static_cast<double>(n) * rev;
  x -= floor(x);
  const float th = static_cast<float>(x * 6.283185307179586476925286766559);
  float s, c;
  sincosf(th, &s, &c);
  return make_float2(c, s);
}

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Round two floats to bfloat16 (nearest even); `a` goes to the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Round two floats to IEEE half (nearest even); `a` goes to the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16_lo(uint32_t u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u >> 16)));
}

// Rotate the interleaved channel pair held in one 32-bit bf16x2 word.
__device__ __forceinline__ uint32_t rotate_pair(uint32_t u, float2 ph) {
  const float x0 = bf_lo(u), x1 = bf_hi(u);
  return pack_bf16x2(x0 * ph.x - x1 * ph.y, x0 * ph.y + x1 * ph.x);
}

// ---- FP8 (OCP e4m3) pool chunks: 2048 bytes of codes, then 16 int8 exponents ----
constexpr int kChunk8 = LAZYATTN_FP8_CHUNK_BYTES;
static_assert(kChunk8 == 16 * 128 + 16, "FP8 chunk = codes of 16 x 128 values + 16 exponents");

// Two e4m3 codes (the low or high 16 bits of w) as floats; exact.  `hi` must
// fold to a constant (the conversion's word select is an immediate).
__device__ __forceinline__ float2 fp8x2_to_f32(uint32_t w, bool hi) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  const f2v r = hi ? __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true)
                   : __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  return make_float2(r.x, r.y);
}
// Two e4m3 codes as a bf16x2 word; exact (every e4m3 value is a bf16 value).
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, false));
}
// Rotate the channel pair of two e4m3 codes; rounds once, to bf16.
__device__ __forceinline__ uint32_t rotate_fp8_pair(uint32_t w, bool hi, float2 ph) {
  const float2 x = fp8x2_to_f32(w, hi);
  return pack_bf16x2(x.x * ph.x - x.y * ph.y, x.x * ph.y + x.y * ph.x);
}
// 2^e for the int8 exponent in byte b of w.
__device__ __forceinline__ float exp_scale(uint32_t w, int b) {
  return __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(static_cast<int8_t>((w >> (8 * b)) & 0xffu)));
}

struct EntryInfo {
  uint32_t blk;
  int32_t start;
  int32_t len;
};

// Decode table entry e of a request: block id, logical start and valid length
// (next entry's start, or the context length for the last entry).  The words
// are read through the constant address space: tables are never written while
// a kernel runs, and a wave-uniform index then always makes a scalar load,
// whatever stores the kernel holds.
typedef const __attribute__((address_space(4))) uint64_t* const_words;
__device__ __forceinline__ EntryInfo entry_info(const uint64_t* row_ptr, int e, int n_ent, int ctx) {
  const const_words row = (const_words)row_ptr;   // an address-space cast
  const uint64_t w = row[e];
  EntryInfo r;
  r.blk = word_block(w);
  r.start = static_cast<int32_t>(word_start(w));
  const int nxt = (e + 1 < n_ent) ? static_cast<int32_t>(word_start(row[e + 1])) : ctx;
  r.len = nxt - r.start;
  return r;
}

__device__ __forceinline__ float alibi_slope(const float* slopes, int h, int Hq) {
  return slopes ? slopes[h] : exp2f(-8.0f * static_cast<float>(h + 1) / static_cast<float>(Hq));
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Prefill, bf16, MFMA.
//
// Work-group = 8 waves (two per SIMD) = 256 query rows: the G heads of one
// KV group at m_q = 256 / G consecutive positions (row rho -> position
// rho / G, head rho % G).  Each wave owns 32 rows, one 32-column MFMA tile.
// A key tile is four table entries (64 key slots).  Per tile and wave:
//   S^T (keys x rows) = K~ (keys x D) . Q~^T       16  32x32x16 MFMA
//   P = 2^(S - m), rounded to bf16                 (base 2, scale folded into Q~)
//   O^T (D x rows)   += V^T (D x keys) . P^T       16  32x32x16 MFMA
// The softmax denominator sums exactly the bf16 weights that enter P.V: each
// lane accumulates its 8-key slices with v_dot2_f32_bf16 against ones, and the
// two key halves (lanes c, c + 32) are added at the end.
//
// Key order.  Within a 32-key half (tau) of the tile, S^T row i holds the key
// that `krow_of` maps to it, chosen so that the accumulator leaves each lane,
// for its query column, keys 8h..8h+7 of two consecutive entries
// (h = lane / 32) in register order.  Those eight weights are exactly a P^T
// operand slice, so P never leaves registers, and the matching V^T operand
// is 8 consecutive keys of one channel: 16 bytes of the pool's own
// channel-major block layout, copied to LDS unchanged.
//
// Reference maximum.  Scores are formed relative to a fixed per-row
// reference m that enters the QK chain as the MFMA's initial accumulator
// (-m): the exact maximum of the row over the work-group's first key tile.
// Numerator and denominator share it, so the result is exact whatever m is,
// as long as 2^(s - m) stays finite; a row sum above 2^64 flags the rare case
// where a later score outgrew m by that much, and the work-group then redoes
// its rows with m set to the exact row maximum over all its keys (one QK-only
// pass first).  ALiBi, whose bias grows toward the diagonal, walks the key
// tiles nearest-first, so the first tile's maximum is taken where the bias is
// largest; it redoes only on the same out-of-range row sums.
//
// Staging.  Wave w stages rows 8 (w % 2) .. + 7 of entry w / 2 of the next
// tile: lane l loads channel pair l of those 8 key rows (4 B each) and
// 2 x 16 B of V one iteration ahead, rotates the keys by R(t - p0) (phase
// R(start - p0 + row) stepped by R(1) per row) between the QK products, and
// writes K~ and V into the other LDS buffer (keys that need no per-row work,
// in the rotation-free, ALiBi and keys-turned-once kernels, move as two 16-byte
// pieces of 4 rows per lane instead).  One barrier per tile.  Table words are fetched three tiles ahead
// and decoded per wave with lane reads.  With the key range split, each
// split writes its output divided by its own row sum, as IEEE half (so split
// calls need |V| <= 65504), and fp32 (m, l); the merge kernel combines them.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// e^{i n f} with f = 2 pi rev, the angle reduced to a fraction of a turn in
// double; the hardware sine/cosine take their argument in turns.
__device__ __forceinline__ float2 unit_phase_turns(int n, double rev) {
  double x = static_cast<double>(n) * rev;
  x -= floor(x);
  const float t = static_cast<float>(x);
  return make_float2(__builtin_amdgcn_cosf(t), __builtin_amdgcn_sinf(t));
}

// The same for a small offset 0 <= n < 2^8 (a query row inside its tile), with
// the angle formed in float: n rev <= 41 turns, so its error stays below
// 41 * 2^-23 turns (3e-5 rad), far under the bf16 rounding of the rotated row.
__device__ __forceinline__ float2 unit_phase_turns_small(int n, double rev) {
  float x = static_cast<float>(n) * static_cast<float>(rev);
  x -= floorf(x);
  return make_float2(__builtin_amdgcn_cosf(x), __builtin_amdgcn_sinf(x));
}

struct PrefillArgs {
  const uint16_t* q;
  const int32_t* cu_q;
  const uint16_t* kpool;
  const uint16_t* vpool;
  const uint64_t* tables;
  const int32_t* n_ent;
  const int32_t* ctx;
  const int32_t* frames;         // [R][max_entries] frame starts (document-local frames) or NULL
  const int32_t* order;          // [R] the order in which work-groups take the requests, or NULL
  const float* alibi;
  uint16_t* out;
  uint16_t* o_part;              // split partials: o / l in fp16 [splits][rows][Hq][D]
  float* ml_part;                // and (m, l) [splits][rows][Hq][2]
  const uint16_t* kturned;       // keys turned once (kPeKeysTurned): [R][Hkv][max_entries][16][D]
  int32_t Hq, Hkv, G, max_entries, total_q, m_q, eps, splits;
  int32_t n_qt;                  // query tiles per request (the grid's x extent is n_qt * splits)
  int32_t xcd_units;             // nonzero: the query tiles of one (split, request, KV head) all run on one XCD
  int32_t exact;                 // nonzero: always take the two-pass exact-maximum route
  float scale_log2;
  RopeRev rope;
};

constexpr int kPD = 128;                 // head dim of the bf16 kernels
// Kernel instantiation for RoPE over a pool in document-local frames: a key
// row at logical position t is stored as R(t - F) k, F its entry's frame start
constexpr int kPeFramed = 3;
// Kernel instantiation for RoPE over keys already turned once per request by
// R(t - c), c = the request's first new position (turn_keys_kernel): the
// attention kernel turns only the queries, by R(m - c), and stages the keys
// as the rotation-free kernel does
constexpr int kPeKeysTurned = 4;
constexpr int kPrefillThreads = 512;    // threads per prefill work-group
constexpr int kKS = kPD + 8;             // K~ row stride in bf16 (272 B: conflict-free 16 B reads)
// V of one entry in LDS: two planes [token half][channel][8 tokens], so that an
// MFMA operand read (8 tokens of consecutive channels per lane) covers
// contiguous bytes; the second plane sits 64 B off a 128 B boundary, which
// puts the even and odd lanes of a staging write on different banks
constexpr int kVH = kPD * 8 + 32;        // plane stride in bf16 (2112 B)
constexpr int kVEs = 2 * kVH;            // entry stride in bf16
constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64: larger row sums redo with the exact maximum
constexpr float kSumFloor = 5.42101086242752217e-20f;  // 2^-64: a row with a visible key and a smaller sum redoes too

// LDS row of tile-local key (entry E, row rho) in the K~ buffer (S^T row order)
__device__ __forceinline__ int krow_of(int E, int rho) {
  return 16 * E + 8 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
}

template <int PE, int KV8>
__global__ __launch_bounds__(kPrefillThreads) void prefill_bf16_kernel(const PrefillArgs A) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][64 * kKS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][4 * kVEs];
  __shared__ int redo_s;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ws = __builtin_amdgcn_readfirstlane(wave);
  const int c = lane & 31, h = lane >> 5;
  // grid (query tile and split, request, KV head), the query tile fastest: the
  // work-groups of one request follow each other, in the given request order
  int qt = blockIdx.x % A.n_qt, split = blockIdx.x / A.n_qt;
  int kvh = blockIdx.z;
  int r = blockIdx.y;
  if (A.xcd_units) {
    // work-group L of the dispatch order runs on XCD L % 8.  With U units
    // (split, request, KV head) a multiple of 8, XCD x takes the units u = x,
    // x + 8, ... with all query tiles of each, so that those tiles, which read
    // the same keys, share one L2; with U = 1, 2 or 4 (the host sets this only
    // when the tiles divide evenly), unit x % U is spread over the 8 / U XCDs
    // x % U, x % U + U, ... instead of all eight
    const int L = static_cast<int>(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    const int k = L >> 3, x = L & 7;
    const int U = A.splits * static_cast<int>(gridDim.y) * static_cast<int>(gridDim.z);
    int u;
    if (U % 8 == 0) {
      u = x + 8 * (k / A.n_qt);
      qt = k % A.n_qt;
    } else {
      u = x % U;
      qt = x / U + (8 / U) * k;
    }
    split = u % A.splits;
    r = (u / A.splits) % static_cast<int>(gridDim.y);
    kvh = u / (A.splits * static_cast<int>(gridDim.y));
  }
  if (A.order) {
    const int o = A.order[r];
    r = (o >= 0 && o < static_cast<int>(gridDim.y)) ? o : r;
  }
  const int q0 = A.cu_q[r];
  const int q_len = A.cu_q[r + 1] - q0;
  const int m0 = qt * A.m_q;
  if (m0 >= q_len) return;
  const int L = A.ctx[r];
  const int ne = min(A.n_ent[r], A.max_entries);
  const int p0 = L - q_len + m0;                      // position of the tile's first row
  const int mq = min(A.m_q, q_len - m0);
  const int p_last = p0 + mq - 1;
  const uint64_t* trow = A.tables + static_cast<size_t>(r) * A.max_entries;
  const int e_begin = split * A.eps;
  const int e_end = min(ne, e_begin + A.eps);
  const int G = A.G, Hq = A.Hq, Hkv = A.Hkv;

  // Entries past the last query position contribute nothing: stop before them.
  // Usually the split's last entry is visible already; otherwise a 64-way
  // vector search over table words finds the first invisible entry.
  int e_stop = max(e_begin, e_end);
  if (e_end > e_begin && static_cast<int>(word_start(trow[e_end - 1])) > p_last) {
    int lo = e_begin, hi = e_end - 1;               // start(hi) > p_last; all before lo are visible
    while (lo < hi) {
      const int stride = (hi - lo + 63) >> 6;
      const int e = lo + lane * stride;
      const bool past = (e < hi) ? static_cast<int>(word_start(trow[e])) > p_last : true;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(past);
      if (bal == 0) {                              // all 64 probes are visible and below hi
        lo = lo + 63 * stride + 1;
        continue;
      }
      const int k = __builtin_ctzll(bal);
      if (k == 0) {
        hi = lo;
      } else {
        const int ek = min(lo + k * stride, hi);
        lo = lo + (k - 1) * stride + 1;
        hi = ek;
      }
    }
    e_stop = lo;
  }
  const int T = (e_stop - e_begin + 3) >> 2;          // key tiles of this work-group
  const int st_first = (T > 0) ? static_cast<int>(word_start(trow[e_begin])) : L;   // first key position
  // ALiBi walks the tiles nearest-first: the first tile then holds the keys of
  // largest bias, whose maximum is the softmax reference (its key weighs exactly
  // 1, as on the exact route); the bias only lowers the scores of later tiles
  constexpr bool kNearestFirst = (PE == LAZYATTN_PE_ALIBI);
  auto tile_e0 = [&](int j) { return e_begin + 4 * (kNearestFirst ? (T - 1 - j) : j); };

  // ---- this lane's query row: column c of the wave's 32-row tile -------------------
  constexpr int NT = 1;
  int p_row[NT], tok[NT], head[NT];
  bool row_ok[NT];
  float slope[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rho = 32 * wave + 32 * nt + c;
    const int m = rho / G;
    row_ok[nt] = m < mq;
    p_row[nt] = p0 + m;
    tok[nt] = q0 + m0 + m;
    head[nt] = kvh * G + (rho - m * G);
    slope[nt] = (PE == LAZYATTN_PE_ALIBI) ? alibi_slope(A.alibi, head[nt], Hq) * kLog2e : 0.0f;
  }

  // Where a tile's staging work goes.  Without per-row work on the staged keys
  // (no rotation, no FP8 conversion) the QK products leave issue slots free,
  // and the staging is spread among them (the rotation-free and ALiBi kernels
  // run 3-8 % faster than with it after the products).  Otherwise those slots
  // hold the rotation, and the staging stays between the QK and P.V phases,
  // where it measured fastest.
  constexpr bool kTurned = PE == kPeKeysTurned;
  constexpr bool kStageEarly = !KV8 && (PE == LAZYATTN_PE_NONE || PE == LAZYATTN_PE_ALIBI || kTurned);

  // ---- table words: lanes x = 0..4 (mod 8) hold word e0 + x of a tile ------------
  // Where the staging work is spread among the QK products (kStageEarly) every
  // lane loads, at an index clamped into the table, so that the load is not
  // predicated (no branch), and entry_of ignores the words past the table's
  // end; otherwise a lane past the end holds the sentinel start L (and the
  // compiler predicates the load).  Nearest-first: tiles past the last (j >= T)
  // lie below e_begin.
  const uint64_t sentinel = static_cast<uint64_t>(static_cast<uint32_t>(L)) << 32;   // start = L
  auto load_words = [&](int j) -> uint64_t {
    const int x = lane & 7;
    const int e = tile_e0(j) + x;
    const uint64_t w = trow[kNearestFirst ? max(min(e, ne - 1), 0) : min(e, ne - 1)];
    if (kStageEarly) return w;
    return (x < 5 && e < ne && (!kNearestFirst || e >= e_begin)) ? w : sentinel;
  };
  // entry x of the tile whose words are in wv: (block, start, length); past the
  // split's last entry the length is 0 and the start L
  auto entry_of = [&](uint64_t wv, int j, int x, int& blk, int& st, int& ln) {
    const uint32_t lo_w = static_cast<uint32_t>(wv), hi_w = static_cast<uint32_t>(wv >> 32);
    const int b = __builtin_amdgcn_readlane(static_cast<int>(lo_w), x);
    const int s0 = __builtin_amdgcn_readlane(static_cast<int>(hi_w), x);
    const int s1w = __builtin_amdgcn_readlane(static_cast<int>(hi_w), x + 1);
    const int e = tile_e0(j) + x;
    const int s1 = (!kStageEarly || e + 1 < ne) ? s1w : L;   // the next entry's start, or the context's end
    const bool valid = e < e_stop && (!kNearestFirst || e >= e_begin);
    blk = valid ? b : 0;
    st = valid ? s0 : L;
    ln = valid ? s1 - s0 : 0;
  };
  // where the keys of entry x of tile j are read, in 4 KiB (16 x D) chunks: the
  // pool's (block, KV head) chunk, or (keys turned once) the request's own
  // turned copy of the entry for this KV head, the split's first entry
  // standing in past the split's end
  auto k_index = [&](int j, int x, int blk) -> size_t {
    if constexpr (!kTurned) return static_cast<size_t>(static_cast<uint32_t>(blk)) * Hkv + kvh;
    const int e = tile_e0(j) + x;
    return (static_cast<size_t>(r) * Hkv + kvh) * A.max_entries + static_cast<size_t>(e < e_stop ? e : e_begin);
  };

  // frame starts (framed pool): lanes x = 0..3 (mod 8) hold entry e0 + x of a tile
  const int32_t* frow = A.frames + (PE == kPeFramed ? static_cast<size_t>(r) * A.max_entries : 0);
  auto load_frames = [&](int j) -> int {
    const int x = lane & 7;
    const int e = e_begin + 4 * j + x;
    return (PE == kPeFramed && x < 4 && e < ne) ? frow[e] : 0;
  };

  // ---- staging: wave w handles rows 8 part .. 8 part + 7 of entry E = w / 2 --------
  // K: lane l holds channel pair l of the 8 key rows (4 B each; with early
  // staging, 8 channels of rows l / 16 and l / 16 + 4 instead); V: lane l holds
  // keys 8 (l % 2) .. + 7 of channels 64 part + 32 cc + l / 2, cc = 0, 1
  const int E_own = ws >> 1, part = ws & 1;
  // this lane's channel-pair frequency (turns per position), read once
  const double rev_l = (PE == LAZYATTN_PE_ROPE || PE == kPeFramed) ? A.rope.rev[lane] : 0.0;
  float2 r1 = make_float2(1.f, 0.f);               // R(1) at this lane's pair
  if (PE == LAZYATTN_PE_ROPE) r1 = unit_phase(1, rev_l);
  // The phases of a lane's 8 consecutive key rows: R(a + 1) = R(a) R(1), then
  // R(a + k + 1) = 2 cos(f) R(a + k) - R(a + k - 1), one fused multiply-add per
  // component instead of a complex product.  The rounding of 2 cos(f) shifts the
  // frequency the recurrence follows, so its error grows about as k^2: over the
  // 8 rows it stays below 3e-6 on unit phases, far under the bf16 rounding of
  // the rotated row.
  const float two_cos = 2.0f * r1.x;
  auto next_phase = [&](int k, float2& cur, float2& prev) {
    if (k == 0) {
      prev = cur;
      cur = cmul(cur, r1);
    } else {
      const float2 nx = make_float2(fmaf(two_cos, cur.x, -prev.x), fmaf(two_cos, cur.y, -prev.y));
      prev = cur;
      cur = nx;
    }
  };
  uint32_t kr[8];
  uint4 vr[2];
  // FP8 pool: kr[k] holds the two codes of row 8 part + k (low 16 bits), vr[cc].xy
  // the 8 codes, and kx / vx the exponents of the 8 key rows / 8 tokens
  uint2 kx = make_uint2(0, 0), vx = make_uint2(0, 0);
  // entries past the split's end (length 0) read block 0: their keys are
  // masked out of the scores and their V rows zeroed when staged
  auto load_k = [&](size_t base) {
    if (KV8) {
      const uint8_t* kc = reinterpret_cast<const uint8_t*>(A.kpool) + base * kChunk8;
      const uint16_t* kp = reinterpret_cast<const uint16_t*>(kc + 8 * part * kPD) + lane;
#pragma unroll
      for (int k = 0; k < 8; ++k) kr[k] = kp[k * (kPD / 2)];
      kx = *reinterpret_cast<const uint2*>(kc + 16 * kPD + 8 * part);
    } else if (kStageEarly) {
      // no per-row work on these keys: two 16-byte loads, rows 8 part + 4 i + lane / 16
      // (i = 0, 1), channels 8 (lane % 16) .. + 7, into kr[4 i .. 4 i + 3]
      const uint16_t* ksrc = kTurned ? A.kturned : A.kpool;
      const uint16_t* kp = ksrc + base * (kBlock * kPD) + (8 * part + (lane >> 4)) * kPD + 8 * (lane & 15);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(kp + 4 * i * kPD);
        kr[4 * i] = v.x;
        kr[4 * i + 1] = v.y;
        kr[4 * i + 2] = v.z;
        kr[4 * i + 3] = v.w;
      }
    } else {
      const uint32_t* kp = reinterpret_cast<const uint32_t*>(A.kpool + base * (kBlock * kPD) + 8 * part * kPD) + lane;
#pragma unroll
      for (int k = 0; k < 8; ++k) kr[k] = kp[k * (kPD / 2)];
    }
  };
  auto load_v = [&](int blk) {
    const size_t base = static_cast<size_t>(static_cast<uint32_t>(blk)) * Hkv + kvh;
    if (KV8) {
      const uint8_t* vc = reinterpret_cast<const uint8_t*>(A.vpool) + base * kChunk8;
      const uint8_t* vp = vc + (64 * part + (lane >> 1)) * kBlock + 8 * (lane & 1);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const uint2 w = *reinterpret_cast<const uint2*>(vp + 32 * cc * kBlock);
        vr[cc] = make_uint4(w.x, w.y, 0u, 0u);
      }
      vx = *reinterpret_cast<const uint2*>(vc + 16 * kPD + 8 * (lane & 1));
    } else {
      const uint16_t* vp = A.vpool + base * (kPD * kBlock) + (64 * part + (lane >> 1)) * kBlock + 8 * (lane & 1);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) vr[cc] = *reinterpret_cast<const uint4*>(vp + 32 * cc * kBlock);
    }
  };
  auto load_kv = [&](size_t kb, int blk) {
    load_k(kb);
    load_v(blk);
  };
  // FP8: the staged key row k (its codes, times 2^exponent) as bf16, turned by ph
  // for RoPE; V codes times their tokens' 2^exponent as bf16.  Exact but for
  // the rotation's rounding.
  auto key_fp8 = [&](int k, float2 ph) -> uint32_t {
    const float sc = exp_scale(k < 4 ? kx.x : kx.y, k & 3);
    if (PE == LAZYATTN_PE_ROPE || PE == kPeFramed) {
      const float2 x = fp8x2_to_f32(kr[k], false);
      const float x0 = x.x * sc, x1 = x.y * sc;
      return pack_bf16x2(x0 * ph.x - x1 * ph.y, x0 * ph.y + x1 * ph.x);
    }
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(kr[k]), sc, false));
  };
  auto convert_v8 = [&]() {
    float sc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) sc[t] = exp_scale(t < 4 ? vx.x : vx.y, t & 3);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const float2 a = fp8x2_to_f32(vr[cc].x, false), b = fp8x2_to_f32(vr[cc].x, true);
      const float2 c2 = fp8x2_to_f32(vr[cc].y, false), d = fp8x2_to_f32(vr[cc].y, true);
      vr[cc] = make_uint4(pack_bf16x2(a.x * sc[0], a.y * sc[1]), pack_bf16x2(b.x * sc[2], b.y * sc[3]),
                          pack_bf16x2(c2.x * sc[4], c2.y * sc[5]), pack_bf16x2(d.x * sc[6], d.y * sc[7]));
    }
  };
  // zero V rows past the entry's length (their weights are 0, but the pool's
  // padding may hold anything)
  auto mask_v = [&](int ln) {
    const int k0 = 8 * (lane & 1);
    uint32_t keep[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      keep[k] = ((k0 + 2 * k < ln) ? 0xffffu : 0u) | ((k0 + 2 * k + 1 < ln) ? 0xffff0000u : 0u);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
      vr[cc] = make_uint4(vr[cc].x & keep[0], vr[cc].y & keep[1], vr[cc].z & keep[2], vr[cc].w & keep[3]);
  };
  // write the staged K~ and V into LDS buffer b
  auto stage_write_k = [&](int b) {
    if constexpr (kStageEarly) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<uint4*>(&Ks[b][krow_of(E_own, 8 * part + 4 * i + (lane >> 4)) * kKS + 8 * (lane & 15)]) =
            make_uint4(kr[4 * i], kr[4 * i + 1], kr[4 * i + 2], kr[4 * i + 3]);
    } else {
      uint32_t* kdst = reinterpret_cast<uint32_t*>(Ks[b]) + lane;
#pragma unroll
      for (int k = 0; k < 8; ++k) kdst[krow_of(E_own, 8 * part + k) * (kKS / 2)] = kr[k];
    }
  };
  auto stage_write_v = [&](int b) {
    uint16_t* vdst = Vs[b] + E_own * kVEs + (lane & 1) * kVH;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
      *reinterpret_cast<uint4*>(&vdst[(64 * part + 32 * cc + (lane >> 1)) * 8]) = vr[cc];
  };
  auto stage_write = [&](int b) {
    stage_write_k(b);
    stage_write_v(b);
  };

  // ---- query: rotated by R(m - p0) (R(m - c) for keys turned once), scaled by ----
  // ---- scale*log2(e), rounded to bf16 --------------------------------------------
  // B operand of k-step kk: channels 16 kk + 8 h .. + 7 of the row
  bf16x8 qf[8 * NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (row_ok[nt])
        raw = *reinterpret_cast<const uint4*>(A.q + (static_cast<size_t>(tok[nt]) * Hq + head[nt]) * kPD + 16 * kk +
                                              8 * h);
      uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float x0 = bf_lo(w4[jj]), x1 = bf_hi(w4[jj]);
        if (PE == LAZYATTN_PE_ROPE || PE == kPeFramed || kTurned) {
          // R(m - p0) against keys turned by R(t - p0); R(m - c) against keys turned once
          const float2 ph = kTurned ? unit_phase_turns(p_row[nt] - (L - q_len), A.rope.rev[8 * kk + 4 * h + jj])
                                    : unit_phase_turns_small(p_row[nt] - p0, A.rope.rev[8 * kk + 4 * h + jj]);
          const float y0 = x0 * ph.x - x1 * ph.y;
          const float y1 = x0 * ph.y + x1 * ph.x;
          x0 = y0;
          x1 = y1;
        }
        w4[jj] = pack_bf16x2(x0 * A.scale_log2, x1 * A.scale_log2);
      }
      qf[8 * nt + kk] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
    }

  f32x16 O[4][NT];
  float lsum[NT];                                    // this lane's part of the row sum (keys 8h..8h+7)
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  float m_ref[NT] = {0.f};                           // reference per row (raw score units)
  f32x16 negm[NT];

  // Turn (RoPE, frames) or convert (FP8) staged key row k; called between QK
  // products so that the work hides under them
  auto stage_row = [&](int k, float2& ph, float2& pq) __attribute__((always_inline)) {
    if (PE == LAZYATTN_PE_ROPE) {
      kr[k] = KV8 ? key_fp8(k, ph) : rotate_pair(kr[k], ph);
      if (k < 7) next_phase(k, ph, pq);
    } else if (KV8) {
      kr[k] = key_fp8(k, ph);                 // framed: turned by ph; else converted
    } else if (PE == kPeFramed) {
      kr[k] = rotate_pair(kr[k], ph);
    }
    if (k == 3 && KV8) convert_v8();
    // keep the row's work between the products around it (the compiler would
    // otherwise sink it to the LDS write)
    asm volatile("" : "+v"(kr[k]));
  };

  // One pass over the key tiles.  maxpass: scores only, folded into the exact
  // row maximum mx[].  Otherwise P.V with the reference m_ref (taken from the
  // first tile when `fresh`).
  float mx[NT] = {kNegInf};
  auto pass = [&](const bool maxpass, const bool fresh) __attribute__((always_inline)) {
    uint64_t wv0 = load_words(0), wv1 = load_words(1), wv2 = load_words(2);
    int fv1 = 0, fv2 = 0;
    {
      int blk, st, ln;
      entry_of(wv0, 0, E_own, blk, st, ln);
      const size_t kb0 = k_index(0, E_own, blk);
      int fv0 = 0;
      if (PE == kPeFramed) {
        fv0 = load_frames(0);
        fv1 = load_frames(1);
        fv2 = load_frames(2);
      }
      load_kv(kb0, blk);
      if (PE == LAZYATTN_PE_ROPE) {
        float2 ph = unit_phase_turns(st - p0 + 8 * part, rev_l), pq;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          kr[k] = KV8 ? key_fp8(k, ph) : rotate_pair(kr[k], ph);
          if (k < 7) next_phase(k, ph, pq);
        }
      } else if (KV8 && PE != kPeFramed) {
#pragma unroll
        for (int k = 0; k < 8; ++k) kr[k] = key_fp8(k, make_float2(1.f, 0.f));
      }
      if (KV8) convert_v8();
      if (PE == kPeFramed) {
        // every row of the entry turns by the same R(F - p0)
        const float2 ph = unit_phase_turns(__builtin_amdgcn_readlane(fv0, E_own) - p0, rev_l);
#pragma unroll
        for (int k = 0; k < 8; ++k) kr[k] = KV8 ? key_fp8(k, ph) : rotate_pair(kr[k], ph);
      }
      if (ln < kBlock) mask_v(ln);
      stage_write(0);
      entry_of(wv1, 1, E_own, blk, st, ln);
      load_kv(k_index(1, E_own, blk), blk);
    }
    __syncthreads();
    for (int i = 0; i < T; ++i) {
      // stage tile i + 1 (loaded during the previous iteration) between the
      // products that form S for tile i; buffer (i + 1) & 1 is free since the
      // barrier that ended iteration i - 1
      int nblk, nst, nln;
      entry_of(wv1, i + 1, E_own, nblk, nst, nln);
      const uint16_t* kb = Ks[i & 1];
      int st[4], ln[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        int b_unused;
        entry_of(wv0, i, x, b_unused, st[x], ln[x]);
      }
      // every key of the tile is a whole block's and visible to every row
      const bool full = (ln[0] == kBlock) && (ln[1] == kBlock) && (ln[2] == kBlock) && (ln[3] == kBlock) &&
                        (st[3] + kBlock - 1 <= p0);
      float2 ph = make_float2(1.f, 0.f), pq = ph;
      if (PE == LAZYATTN_PE_ROPE) ph = unit_phase_turns(nst - p0 + 8 * part, rev_l);
      if (PE == kPeFramed) ph = unit_phase_turns(__builtin_amdgcn_readlane(fv1, E_own) - p0, rev_l);
      uint64_t wv3;
      int fv3;
      f32x16 S[2][NT];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) S[tau][nt] = negm[nt];
      // K~ operands are read one k-step ahead of their products
      bf16x8 ak[2][2];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) ak[0][tau] = *reinterpret_cast<const bf16x8*>(&kb[(32 * tau + c) * kKS + 8 * h]);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if (kk + 1 < 8) {
#pragma unroll
          for (int tau = 0; tau < 2; ++tau)
            ak[(kk + 1) & 1][tau] =
                *reinterpret_cast<const bf16x8*>(&kb[(32 * tau + c) * kKS + 16 * (kk + 1) + 8 * h]);
        }
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) S[tau][nt] = mfma32x32x16(ak[kk & 1][tau], qf[8 * nt + kk], S[tau][nt]);
        stage_row(kk, ph, pq);
      }
      // Staging of the next tiles, then the words of tile i + 3 before the loads
      // of tile i + 2 (in this order, the copies of the word registers at the
      // end of the tile wait for the word load only, not for the K/V loads
      // issued after it).
      int lblk, lst, lln;
      if constexpr (kStageEarly) {
        // K~ of tile i + 1 (never masked: the scores of padded keys are) and the
        // K loads here, V at the P.V products: no branch separates this work
        // from the QK products, so that the scheduler spreads it among them
        stage_write_k((i + 1) & 1);
        entry_of(wv2, i + 2, E_own, lblk, lst, lln);
        wv3 = load_words(i + 3);
        fv3 = load_frames(i + 3);
        load_k(k_index(i + 2, E_own, lblk));
      } else {
        // rare: only entries shorter than a block need their padding zeroed
        if (__builtin_expect(nln < kBlock, 0)) mask_v(nln);
        stage_write((i + 1) & 1);
        entry_of(wv2, i + 2, E_own, lblk, lst, lln);
        wv3 = load_words(i + 3);
        fv3 = load_frames(i + 3);
        load_kv(k_index(i + 2, E_own, lblk), lblk);
      }

      // register r of half tau: key row 8 h + (r % 8) of entry 2 tau + r / 8
      if (PE == LAZYATTN_PE_ALIBI) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int t = st[2 * tau + (rr >> 3)] + 8 * h + (rr & 7);
              S[tau][nt][rr] -= slope[nt] * static_cast<float>(p_row[nt] - t);
            }
      }
      // rare: a tile with padded or invisible keys, or a staged entry shorter
      // than a block (its V padding is zeroed: the pool may hold anything there)
      if (__builtin_expect(!full || (kStageEarly && nln < kBlock), 0)) {
        if (kStageEarly && nln < kBlock) mask_v(nln);
        if (!full) {
#pragma unroll
          for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int E = 2 * tau + (rr >> 3), kr_ = 8 * h + (rr & 7);
              const int t = st[E] + kr_;
              const bool live = kr_ < ln[E];
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) S[tau][nt][rr] = (live && t <= p_row[nt]) ? S[tau][nt][rr] : kNegInf;
            }
        }
      }
      if (maxpass || (fresh && i == 0)) {
        // row maximum of this tile (lanes c and c + 32 hold the two key halves)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float lm = kNegInf;
#pragma unroll
          for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int rr = 0; rr < 16; rr += 2) lm = fmaxf(lm, fmaxf(S[tau][nt][rr], S[tau][nt][rr + 1]));
          lm = fmaxf(lm, __shfl_xor(lm, 32));
          if (maxpass) {
            mx[nt] = fmaxf(mx[nt], lm);
          } else {
            const float mr = (lm == kNegInf) ? 0.f : lm;      // a fully masked row keeps reference 0
            m_ref[nt] = mr;
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) S[tau][nt] -= mr;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) negm[nt][rr] = -mr;
          }
        }
      }
      if constexpr (kStageEarly) {
        // V of tile i + 1, then the V loads of tile i + 2
        stage_write_v((i + 1) & 1);
        load_v(lblk);
      }
      if (!maxpass) {
        // P^T operands (weights of keys 8 h .. 8 h + 7 of entry 2 tau + ks) and
        // O^T += V^T P^T, V of entry E read from its token-half planes;
        // the exponentials of one entry overlap the products of the previous
        const uint16_t* vb = Vs[i & 1];
        // V operands (entry E, channel tile dt: read number 4 E + dt) two reads ahead
        auto vread = [&](int n) {
          return *reinterpret_cast<const bf16x8*>(&vb[(n >> 2) * kVEs + h * kVH + (32 * (n & 3) + c) * 8]);
        };
        bf16x8 av[3];
        av[0] = vread(0);
        av[1] = vread(1);
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 Pk[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              uint32_t pw[4];
#pragma unroll
              for (int k = 0; k < 4; ++k)
                pw[k] = pack_bf16x2(__builtin_amdgcn_exp2f(S[tau][nt][8 * ks + 2 * k]),
                                    __builtin_amdgcn_exp2f(S[tau][nt][8 * ks + 2 * k + 1]));
              Pk[nt] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              const int n = 4 * (2 * tau + ks) + dt;
              if (n + 2 < 16) av[(n + 2) % 3] = vread(n + 2);
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) O[dt][nt] = mfma32x32x16(av[n % 3], Pk[nt], O[dt][nt]);
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const uint4 pw = __builtin_bit_cast(uint4, Pk[nt]);
              lsum[nt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.x), ones2, lsum[nt], false);
              lsum[nt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.y), ones2, lsum[nt], false);
              lsum[nt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.z), ones2, lsum[nt], false);
              lsum[nt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.w), ones2, lsum[nt], false);
            }
          }
      }
      wv0 = wv1;
      wv1 = wv2;
      wv2 = wv3;
      fv1 = fv2;
      fv2 = fv3;
      __syncthreads();
    }
  };

  auto clear_acc = [&]() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) O[dt][nt] = f32x16{};
      lsum[nt] = 0.f;
      negm[nt] = f32x16{};
    }
  };
  clear_acc();
  bool two_pass = A.exact != 0;
  if (T > 0 && !two_pass) {
    pass(false, true);
    // a row sum this large means some score outgrew the first tile's maximum,
    // and one this small (with a visible key) that every weight underflowed:
    // either way, redo the work-group with the exact maximum
    bool bad = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float lt = lsum[nt] + __shfl_xor(lsum[nt], 32);
      const bool visible = st_first <= p_row[nt];
      bad = bad || (row_ok[nt] && (!(lt < kSumLimit) || (visible && !(lt >= kSumFloor))));
    }
    if (tid == 0) redo_s = 0;
    __syncthreads();
    if (__builtin_amdgcn_ballot_w64(bad) && lane == 0) redo_s = 1;
    __syncthreads();
    two_pass = redo_s != 0;
  }
  if (T > 0 && two_pass) {
    clear_acc();                                     // scores of the max pass are raw (reference 0)
    pass(true, false);
    clear_acc();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m_ref[nt] = (mx[nt] == kNegInf) ? 0.f : mx[nt];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) negm[nt][rr] = -m_ref[nt];
    }
    pass(false, false);
  }

  // ---- epilogue ----------------------------------------------------------------
  // row sum = this lane's half + the other key half's (lane c + 32); O register
  // r: channel 32 dt + 8 (r / 4) + 4 h + r % 4
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = lsum[nt] + __shfl_xor(lsum[nt], 32);
    if (!row_ok[nt]) continue;
    const size_t rowoff = static_cast<size_t>(tok[nt]) * Hq + head[nt];
    if (A.splits == 1) {
      const float inv = 1.0f / lt;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          *reinterpret_cast<uint2*>(A.out + rowoff * kPD + 32 * dt + 8 * qq + 4 * h) =
              make_uint2(pack_bf16x2(O[dt][nt][4 * qq] * inv, O[dt][nt][4 * qq + 1] * inv),
                         pack_bf16x2(O[dt][nt][4 * qq + 2] * inv, O[dt][nt][4 * qq + 3] * inv));
    } else {
      // this split's output divided by its own sum (fp16), reference and sum
      const size_t prow = static_cast<size_t>(split) * A.total_q * Hq + rowoff;
      if (lt > 0.f) {
        const float inv = 1.0f / lt;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            *reinterpret_cast<uint2*>(A.o_part + prow * kPD + 32 * dt + 8 * qq + 4 * h) =
                make_uint2(pack_f16x2(O[dt][nt][4 * qq] * inv, O[dt][nt][4 * qq + 1] * inv),
                           pack_f16x2(O[dt][nt][4 * qq + 2] * inv, O[dt][nt][4 * qq + 3] * inv));
      }
      if (h == 0)
        *reinterpret_cast<float2*>(A.ml_part + prow * 2) = make_float2(lt > 0.f ? m_ref[nt] : kNegInf, lt);
    }
  }
}

// ---------------------------------------------------------------------------
// Split merge: out = sum_s w_s (o_s / l_s) / sum_s w_s with w_s = 2^(m_s - M) l_s
// and M = max_s m_s.  Each split's output is stored already divided by its own
// sum, in fp16 (a relative rounding of 2^-11, under the bf16 rounding of the
// result), which halves the partial traffic.  One 16-lane group per (row,
// head), 8 channels (16 bytes) per lane.  Splits are taken CH at a time with
// their loads issued together (nothing is read past the last split); M is the
// running maximum, and what was summed before
// a chunk raised it is rescaled (the order is fixed: reproducible bit for
// bit).  A split with m = -inf (no visible key, or past its request's end)
// weighs 0, and its output, which may never have been written, is dropped by a
// select.
// ---------------------------------------------------------------------------
// CH = splits whose loads are issued together: 16 for calls of more than 4 splits
// (one memory round trip for up to 16), else 4 (fewer registers for the
// bandwidth-bound merges of few splits)
// List mode (list_begin != NULL, shared-run decode): output row idx = r Hq + h
// merges the partials of request r's occurrences, rows list[i] Hq + h for i in
// list_begin[r] .. list_begin[r + 1], in that order.
template <int CH>
__global__ __launch_bounds__(256) void merge_kernel(const uint16_t* o_part, const float* ml_part, uint16_t* out,
                                                    int rows, int splits, const int32_t* list_begin,
                                                    const int32_t* list, int Hq) {
  const int idx = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;                  // channels 8c .. 8c + 7
  if (idx >= rows) return;
  int l0 = 0, hh = 0;
  if (list_begin) {
    const int rq = idx / Hq;
    hh = idx - rq * Hq;
    l0 = list_begin[rq];
    splits = list_begin[rq + 1] - l0;
  }
  float M = kNegInf, lsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += CH) {
    float2 ml[CH];
    uint4 o[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      // past the last split (the row's last occurrence) nothing is read
      ml[j] = make_float2(kNegInf, 0.f);
      o[j] = make_uint4(0u, 0u, 0u, 0u);
      if (s0 + j < splits) {
        const size_t row = list_begin ? static_cast<size_t>(list[l0 + s0 + j]) * Hq + hh
                                      : static_cast<size_t>(s0 + j) * rows + idx;
        ml[j] = *reinterpret_cast<const float2*>(ml_part + row * 2);
        o[j] = *reinterpret_cast<const uint4*>(o_part + row * kPD + 8 * c);
      }
    }
    bool live[CH];
    float mc = kNegInf;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      live[j] = (s0 + j < splits) && (ml[j].x != kNegInf);
      mc = fmaxf(mc, live[j] ? ml[j].x : kNegInf);
    }
    const float Mn = fmaxf(M, mc);
    const float f = (M == kNegInf || Mn == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(M - Mn);
    lsum *= f;
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] *= f;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float w = live[j] ? __builtin_amdgcn_exp2f(ml[j].x - Mn) * ml[j].y : 0.f;
      lsum += w;
      const uint32_t ow[4] = {o[j].x, o[j].y, o[j].z, o[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(w, live[j] ? f16_lo(ow[q]) : 0.f, acc[2 * q]);
        acc[2 * q + 1] = fmaf(w, live[j] ? f16_hi(ow[q]) : 0.f, acc[2 * q + 1]);
      }
    }
    M = Mn;
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  *reinterpret_cast<uint4*>(out + static_cast<size_t>(idx) * kPD + 8 * c) =
      make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                 pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
}

// ---------------------------------------------------------------------------
// Decode, bf16, MFMA, split-K over table entries.
//
// Work-group = 4 waves for one (request, KV head, split); wave w takes
// entries e_begin + w, + 4, ...  Per block (16 keys) a wave computes
//   S^T (16 keys x 16 heads) = K~ (16 x D) . q^T            4 x 16x16x32 MFMA
//   O^T (D x 16 heads)      += V^T (D x 16 keys) . P^T      8 x 16x16x16 MFMA
// with the group's G heads padded to NT tiles of 16 (NT = 2 for groups of 17..32
// heads over a plain content-only pool: every block is read and turned once for
// all of them; over FP8 pools and framed batches such groups run as two
// work-groups of 16 heads instead).  Lane (g, n) loads key
// row n, channels 32g..32g+31 (64 contiguous bytes) and V channel rows
// 16dt + n, keys 4g..4g+3 (8 bytes each); the whole 8 KB block is read once.
// Scores are formed relative to a per-head reference m that enters the QK
// chain as the MFMA's initial accumulator (-m); the reference is raised, and O
// rescaled, only when a score outgrows it by more than 2^8, so the common
// block spends no vector instructions on maxima or rescaling.
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kpool;
  const uint16_t* vpool;
  const uint64_t* tables;
  const int32_t* n_ent;
  const int32_t* ctx;
  const int32_t* frames;         // [R][max_entries] frame starts (document-local frames) or NULL
  const int32_t* order;          // [R] the order in which work-groups take the requests, or NULL
  const float* alibi;
  uint16_t* out;
  uint16_t* o_part;              // split partials: o / l in fp16 [splits][rows][Hq][D]
  float* ml_part;                // and (m, l) [splits][rows][Hq][2]
  int32_t R, Hq, Hkv, G, max_entries, eps, splits;
  int32_t halves;                // 2: groups of 17..32 heads as one work-group per 16-head half (FP8, framed)
  float scale_log2;
  RopeRev rope;
  // shared-run decode (items != NULL): work-group (item, KV head) instead of
  // (split, KV head, request); partials go to the occurrence's slot
  const int32_t* items;          // [n_items][4] {first word, entries, first occurrence, occurrences}
  const uint64_t* words;         // item entries: block, key offset (bits 58..32), length (63..59)
  const int32_t* refs;           // [n_refs][2] {request, p - s}
};

constexpr int kOS = kPD + 4;  // LDS row stride (floats) of the wave-merge buffer
constexpr int kTab = 2048;    // table entries staged in LDS at a time (in the merge buffer's space)
constexpr int kRing = 2;      // entries of a decode wave in registers: one processed, the rest in flight
static_assert(4 * kTab * 4 <= 4 * 16 * kOS * 4, "the staged table fits the wave-merge buffer");
constexpr float kRescaleSlack = 8.0f;   // reference raised only when a score exceeds it by 2^8

template <int PE, int NT, int KV8, int RUNS>
__global__ __launch_bounds__(256, 2) void decode_bf16_kernel(const DecodeArgs A) {
  extern __shared__ __attribute__((aligned(16))) float dsm[];
  float2* bsh = reinterpret_cast<float2*>(dsm);             // [4 waves][kRing][64]
  float* ml_s = dsm + 4 * kRing * 64 * 2;                     // [4][NT*16][2]
  float* o_s = ml_s + 4 * NT * 16 * 2;                        // [4][16][kOS]: one 16-column tile at a time
  float2* rtab = reinterpret_cast<float2*>(o_s + 4 * 16 * kOS);  // [16][64] R(n), RoPE only
  uint4* qs = reinterpret_cast<uint4*>(rtab + 16 * 64);          // [NT][4][64] query fragments (NT > 1)

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int G = A.G, Hq = A.Hq, Hkv = A.Hkv;
  // With halves == 2, groups of more than 16 heads run as two work-groups of 16 heads each over
  // the same entries.  Their linear ids differ by 8, so round-robin dispatch
  // puts them on one XCD at about the same time and the second read of each
  // block hits that XCD's L2: ids 16 j + i and 16 j + 8 + i (i < 8) are the
  // two halves of work item 8 j + i = (split, kvh, request), split fastest.
  int split, kvh, r, half = 0;
  // shared-run item: its words, entries, last entry's length, occurrences
  int run_w0 = 0, run_n = 0, run_ref0 = 0, run_nref = 0;
  constexpr bool runs = RUNS != 0;
  if (runs) {
    // one item per wave: items 4 x .. 4 x + 3 of work-group x (an empty item's
    // wave passes the work-group barrier below, then ends)
    const int w_item = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * 4 + wave);
    const int32_t* it = A.items + static_cast<size_t>(w_item) * 4;
    run_w0 = it[0];
    run_n = it[1];
    run_ref0 = it[2];
    run_nref = it[3];
    split = 0;
    kvh = blockIdx.y;
    r = 0;
  } else if (A.halves == 1) {
    split = blockIdx.x;
    kvh = blockIdx.y;
    r = blockIdx.z;
  } else {
    const int id = blockIdx.x;
    const int item = (id >> 4) * 8 + (id & 7);
    half = (id >> 3) & 1;
    if (item >= A.splits * Hkv * A.R) return;
    split = item % A.splits;
    const int rest = item / A.splits;
    kvh = rest % Hkv;
    r = rest / Hkv;
  }
  if (!runs && A.order) {
    // the requests in the given order (an entry outside 0..R-1 stands for its own index)
    const int o = A.order[r];
    r = (o >= 0 && o < A.R) ? o : r;
  }
  const int hb = 16 * half;                          // first head column of this work-group
  // its head columns; a shared-run item's columns are (occurrence, head) pairs
  const int Gw = runs ? min(16 * NT, run_nref * G) : min(16 * NT, G - hb);
  // key positions are relative to the query (p) or, for a shared-run item, to
  // its first key (the queries carry the rest of the turn)
  const int L = runs ? 0 : A.ctx[r];
  const int p = runs ? 0 : L - 1;
  const int ne = runs ? run_n : A.n_ent[r];
  const uint64_t* trow = A.tables + (runs ? 0 : static_cast<size_t>(r) * A.max_entries);
  const int e_begin = runs ? 0 : split * A.eps;
  const int e_end = runs ? run_n : min(ne, e_begin + A.eps);
  // a split past the request's last entry leaves only an empty (m, l) = (-inf, 0),
  // which the merge skips without reading its output
  if (!runs && A.splits > 1 && e_begin >= ne) {
    if (tid < Gw) {
      const size_t prow = static_cast<size_t>(split) * A.R * Hq + static_cast<size_t>(r) * Hq + kvh * G + hb + tid;
      *reinterpret_cast<float2*>(A.ml_part + prow * 2) = make_float2(kNegInf, 0.f);
    }
    return;
  }

  // Channels of contraction step s held by lane (g, n): c0(s) .. c0(s) + 7 with
  // c0(s) = 32s + 8g for bf16 pools (each of a lane's four 16-byte K loads then
  // covers 64 contiguous bytes of every key row) and 32g + 8s for FP8 pools (a
  // lane's 32 code bytes are contiguous).  Any such assignment works as long as
  // q and K agree; the channel pair of word jj is c0(s) / 2 + jj.
  auto c0 = [&](int s) { return KV8 ? 32 * g + 8 * s : 32 * s + 8 * g; };
  // query fragments: lane (g, n) holds head column nt*16+n, channels c0(s) + 0..7,
  // scaled by scale*log2(e) and rounded to bf16
  // (framed pool: the raw fragments are kept, and qb is formed per frame)
  // (shared-run item: column = (occurrence j, head gg) with j = col / G; its
  // query is request refs[j]'s, turned by R(p - s) at every pair when RoPE)
  bf16x8 qb[NT][4];
  uint4 qraw[NT][4];
  float slope[NT];
  int pcol[NT];                                       // the query's position, relative as the keys'
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + n;
    const bool ok = col < Gw;
    int h = kvh * G + hb + (ok ? col : 0), rq = r;
    int turn = 0;
    pcol[nt] = p;
    if (runs) {
      const int j = ok ? col / G : 0;
      h = kvh * G + (ok ? col - j * G : 0);
      rq = ok ? A.refs[2 * (run_ref0 + j)] : 0;
      turn = ok ? A.refs[2 * (run_ref0 + j) + 1] : 0;
      pcol[nt] = turn;
    }
    slope[nt] = (PE == LAZYATTN_PE_ALIBI) ? alibi_slope(A.alibi, h, Hq) * kLog2e : 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (ok) raw = *reinterpret_cast<const uint4*>(A.q + (static_cast<size_t>(rq) * Hq + h) * kPD + c0(s));
      qraw[nt][s] = raw;
      uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float x0 = bf_lo(w4[jj]), x1 = bf_hi(w4[jj]);
        if (PE == LAZYATTN_PE_ROPE && runs) {
          const float2 ph = unit_phase_turns(turn, A.rope.rev[c0(s) / 2 + jj]);
          const float y0 = x0 * ph.x - x1 * ph.y, y1 = x0 * ph.y + x1 * ph.x;
          x0 = y0;
          x1 = y1;
        }
        w4[jj] = pack_bf16x2(x0 * A.scale_log2, x1 * A.scale_log2);
      }
      qb[nt][s] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
    }
  }
  // Two head tiles (NT > 1): the query fragments, the same for every wave, go to
  // LDS and are read back at each entry instead of holding 32 registers
  if (NT > 1) {
    if (wave == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int s = 0; s < 4; ++s) qs[(nt * 4 + s) * 64 + lane] = __builtin_bit_cast(uint4, qb[nt][s]);
    }
    __syncthreads();
  }
  // R(n) of lane (g, n)'s key row n at pair 16g + i, as rtab[i][lane] (a lane's
  // 16 reads of one entry are then 64 consecutive float2 each); this lane's
  // pair for R(S - p)
  double my_rev = 0.0;
  if (PE == LAZYATTN_PE_ROPE) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q, i = idx >> 6, l = idx & 63;
      const int pair = KV8 ? 16 * (l >> 4) + i : 16 * (i >> 2) + 4 * (l >> 4) + (i & 3);   // c0(i / 4) / 2 + i % 4
      rtab[idx] = unit_phase_turns(l & 15, A.rope.rev[pair]);
    }
    __syncthreads();
  }
  if (PE == LAZYATTN_PE_ROPE || PE == kPeFramed) my_rev = A.rope.rev[lane];
  // This lane's R(n) at its 16 pairs, held in registers: reading them from LDS
  // at each entry put an LDS round trip on every entry's path (the empty asm
  // keeps the compiler from turning the copies back into LDS reads at the uses).
  // A wave of two head tiles (NT = 2) has no registers to spare for them and
  // reads them from LDS; its rotation serves twice the heads.
  float2 rn[16];
  if (PE == LAZYATTN_PE_ROPE && NT == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      rn[i] = rtab[i * 64 + lane];
      asm volatile("" : "+v"(rn[i].x), "+v"(rn[i].y));
    }
  }
  // framed pool: the frame the query fragments qb are currently turned to (none yet)
  int q_frame = 0, q_turns = 0;
  bool q_set = false;

  f32x4 O[8][NT];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // per head column: reference m_run (raw score units, -inf until the first
  // visible key), its finite stand-in m_use, and the running sum
  float m_run[NT], m_use[NT], l_run[NT];
  f32x4 negm[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = kNegInf;
    m_use[nt] = 0.f;
    l_run[nt] = 0.f;
    negm[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // bf16 pool: lane (g, n) holds key row n, channels c0(s)..+7 (k[s]), and V
  // channel rows 16dt+n, tokens 4g..4g+3 (v[dt]).  FP8 pool: lane (g, n) holds
  // the 32 codes of key row n, channels 32g..32g+31 (k[0..1]), the codes of tokens 4g..4g+3 of channel rows 16dt+n (vr[dt].x)
  // and the exponents of key rows / tokens 4g..4g+3 (kr[2].x, kr[2].y)
  auto load_kv = [&](uint32_t blk, uint4 (&k)[4], uint2 (&v)[8]) {
    if (KV8) {
      const size_t chunk = (static_cast<size_t>(blk) * Hkv + kvh) * kChunk8;
      const uint8_t* kc = reinterpret_cast<const uint8_t*>(A.kpool) + chunk;
      const uint8_t* vc = reinterpret_cast<const uint8_t*>(A.vpool) + chunk;
      const uint4* kp = reinterpret_cast<const uint4*>(kc + n * kPD + 32 * g);
      k[0] = kp[0];
      k[1] = kp[1];
      k[2].x = *reinterpret_cast<const uint32_t*>(kc + 16 * kPD + 4 * g);
      k[2].y = *reinterpret_cast<const uint32_t*>(vc + 16 * kPD + 4 * g);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) v[dt].x = *reinterpret_cast<const uint32_t*>(vc + (16 * dt + n) * kBlock + 4 * g);
    } else {
      const uint16_t* kb = A.kpool + (static_cast<size_t>(blk) * Hkv + kvh) * (kBlock * kPD);
#pragma unroll
      for (int s = 0; s < 4; ++s) k[s] = *reinterpret_cast<const uint4*>(kb + n * kPD + c0(s));
      const uint16_t* vb = A.vpool + (static_cast<size_t>(blk) * Hkv + kvh) * (kPD * kBlock);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) v[dt] = *reinterpret_cast<const uint2*>(vb + (16 * dt + n) * kBlock + 4 * g);
    }
  };

  // Entries are processed in the wave-uniform order e_begin + wave + 4k, k = 0, 1,
  // ...  kRing ring slots hold the K/V of the entry being processed and of the
  // next kRing - 1 (in flight); a slot is refilled with the entry kRing places
  // on as soon as its entry is done, so its loads have kRing - 1 entries' time
  // to land and no registers are copied.  Past the wave's last entry a slot
  // reloads that entry (its block is already in L2, and the result is never
  // used): every refill then issues the same loads on every path, so the wait
  // for one slot's data never has to drain the others'.
  //
  // The split's table is staged in LDS by the whole work-group, up to kTab
  // entries at a time: each entry's logical start and end (the next entry's
  // start, or L), block id and (framed pools) frame start.  An entry's
  // fields are then LDS reads, which complete in order: no wait for them
  // involves the K/V loads in flight (table words read with scalar loads would
  // share a counter with the LDS reads and return out of order; read with
  // vector loads, they would share the K/V loads' counter).
  uint4 krb[kRing][4];
  uint2 vrb[kRing][8];
  EntryInfo curb[kRing];
  int frb[kRing];
  const int wv = __builtin_amdgcn_readfirstlane(wave);          // wave-uniform, so the loop branches are scalar
  uint32_t* tst = reinterpret_cast<uint32_t*>(o_s);             // [kTab] logical starts (o_s is free until the merge)
  uint32_t* ten = tst + kTab;                                    // [kTab] logical ends
  uint32_t* tbk = ten + kTab;                                    // [kTab] block ids
  int32_t* tfr = reinterpret_cast<int32_t*>(tbk + kTab);         // [kTab] frame starts
  const int32_t* frow_v = A.frames + (PE == kPeFramed ? static_cast<size_t>(r) * A.max_entries : 0);
  int nk = 0, kl = 0;                                            // this wave's entries in the chunk; next to load
  // a wave's entries in the staged table: wv, wv + 4, ... (the work-group's
  // entries), or its own item's rows 0, 1, ... from row (kTab / 4) wv
  const int tab_base = runs ? wv * (kTab / 4) : wv, tab_step = runs ? 1 : 4;
  auto fetch = [&](EntryInfo& inf, int& fr) {
    const int li = tab_base + tab_step * min(kl, nk - 1);
    inf.blk = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(tbk[li])));
    inf.start = __builtin_amdgcn_readfirstlane(static_cast<int>(tst[li]));
    inf.len = __builtin_amdgcn_readfirstlane(static_cast<int>(ten[li])) - inf.start;
    fr = (PE == kPeFramed) ? __builtin_amdgcn_readfirstlane(tfr[li]) : 0;
    ++kl;
  };
  // RoPE: R(S - p) of a slot's entry at pair l, formed by lane l into the slot's
  // LDS row as soon as the entry's loads are issued, so that the entry's
  // rotation reads it without an LDS round trip on its own path.  A wave's
  // entries are four apart: when the next one starts 64 positions after the
  // previous (four whole blocks on), its phase is the previous one times
  // R(64), for at most 32 steps in a row (rounding then adds at most ~1e-5 to
  // a unit phase, far under the bf16 rounding of the rotated key); otherwise
  // it is formed afresh from the angle reduced in fp64.
  // (a wave that takes its item's entries in order steps by one block: R(16))
  const int ph_step = runs ? kBlock : 4 * kBlock;
  float2 ph_prev = make_float2(1.f, 0.f), r64 = make_float2(1.f, 0.f);
  int st_prev = 0, ph_run = 32;
  if (PE == LAZYATTN_PE_ROPE) r64 = unit_phase(ph_step, my_rev);
  auto put_phase = [&](int sl, int start) {
    if (PE == LAZYATTN_PE_ROPE) {
      float2 ph;
      if (start == st_prev + ph_step && ph_run < 32) {
        ph = cmul(ph_prev, r64);
        ++ph_run;
      } else {
        ph = unit_phase_turns(start - p, my_rev);
        ph_run = 0;
      }
      ph_prev = ph;
      st_prev = start;
      bsh[(wave * kRing + sl) * 64 + lane] = ph;
      __builtin_amdgcn_wave_barrier();
    }
  };
  // one entry, its K/V in k and v (converted in place for FP8)
  auto process = [&](const EntryInfo inf, const int fr, uint4 (&k)[4], uint2 (&v)[8], const int sl)
                     __attribute__((always_inline)) {
      const uint32_t kexp = k[2].x, vexp = k[2].y;
      if (KV8) {
        // FP8 codes to bf16 operands (exact); the exponents scale S and P below
        const uint4 c0 = k[0], c1 = k[1];
        const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        if (PE != LAZYATTN_PE_ROPE) {
  #pragma unroll
          for (int s = 0; s < 4; ++s)
            k[s] = make_uint4(fp8x2_to_bf16x2(cw[2 * s], false), fp8x2_to_bf16x2(cw[2 * s], true),
                              fp8x2_to_bf16x2(cw[2 * s + 1], false), fp8x2_to_bf16x2(cw[2 * s + 1], true));
        }
  #pragma unroll
        for (int dt = 0; dt < 8; ++dt) v[dt] = make_uint2(fp8x2_to_bf16x2(v[dt].x, false), fp8x2_to_bf16x2(v[dt].x, true));
      }

      // ---- framed pool: turn the query to this entry's frame, R(p - F) q ----------
      if (PE == kPeFramed && (!q_set || fr != q_frame)) {
        float2* bw = bsh + (wave * kRing + (q_turns & 1)) * 64;
        bw[lane] = unit_phase_turns(p - fr, my_rev);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  #pragma unroll
        for (int nt = 0; nt < NT; ++nt)
  #pragma unroll
          for (int s = 0; s < 4; ++s) {
            uint32_t w4[4] = {qraw[nt][s].x, qraw[nt][s].y, qraw[nt][s].z, qraw[nt][s].w};
  #pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const float2 ph = bw[c0(s) / 2 + jj];
              const float x0 = bf_lo(w4[jj]), x1 = bf_hi(w4[jj]);
              w4[jj] = pack_bf16x2((x0 * ph.x - x1 * ph.y) * A.scale_log2, (x0 * ph.y + x1 * ph.x) * A.scale_log2);
            }
            qb[nt][s] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
          }
        q_frame = fr;
        q_set = true;
        ++q_turns;
      }

      // ---- rotate the key rows: R(S - p + n) = R(S - p) R(n) ------------------
      bf16x8 ka[4];
      if (PE == LAZYATTN_PE_ROPE) {
        // R(S - p) at pair l, written by lane l when the slot was loaded
        const float2* bw = bsh + (wave * kRing + sl) * 64;
        // two head tiles: R(n) read from LDS at each entry (an opaque lane index
        // keeps the compiler from hoisting the reads into 32 live registers)
        int rl = lane;
        if (NT > 1) asm volatile("" : "+v"(rl));
        if (KV8) {
          // the lane's 32 codes are in k[0..1]
  #pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint32_t c_lo = (s < 2) ? (s == 0 ? k[0].x : k[0].z) : (s == 2 ? k[1].x : k[1].z);
            const uint32_t c_hi = (s < 2) ? (s == 0 ? k[0].y : k[0].w) : (s == 2 ? k[1].y : k[1].w);
            uint32_t w4[4];
  #pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              // pair 16g + 4s + jj
              w4[jj] = rotate_fp8_pair(jj < 2 ? c_lo : c_hi, (jj & 1) != 0,
                                       cmul(bw[c0(s) / 2 + jj], NT == 1 ? rn[4 * s + jj] : rtab[(4 * s + jj) * 64 + rl]));
            }
            ka[s] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
          }
        } else {
  #pragma unroll
          for (int s = 0; s < 4; ++s) {
            uint32_t w4[4] = {k[s].x, k[s].y, k[s].z, k[s].w};
  #pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              w4[jj] = rotate_pair(w4[jj], cmul(bw[c0(s) / 2 + jj],
                                                NT == 1 ? rn[4 * s + jj] : rtab[(4 * s + jj) * 64 + rl]));   // pair 16s + 4g + jj
            }
            ka[s] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
            // two head tiles: one contraction step's phases at a time (registers)
            if (NT > 1) __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
  #pragma unroll
        for (int s = 0; s < 4; ++s) ka[s] = __builtin_bit_cast(bf16x8, k[s]);
      }
      // (the branches below are rare: marked so, their code stays out of the
      // entry's straight-line path)
      if (__builtin_expect(inf.len < kBlock, 0)) {
        // zero V rows past the entry's length (they may hold anything, even NaN)
  #pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          uint32_t a = v[dt].x, b = v[dt].y;
          const int k0 = 4 * g;
          a = ((k0 + 0 < inf.len) ? (a & 0xffffu) : 0u) | ((k0 + 1 < inf.len) ? (a & 0xffff0000u) : 0u);
          b = ((k0 + 2 < inf.len) ? (b & 0xffffu) : 0u) | ((k0 + 3 < inf.len) ? (b & 0xffff0000u) : 0u);
          v[dt] = make_uint2(a, b);
        }
      }

  #pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // scores relative to the reference: the chain starts from -m (FP8: the
        // row's scale multiplies the product first)
        f32x4 S = KV8 ? f32x4{0.f, 0.f, 0.f, 0.f}
                      : (NT == 1 ? negm[nt] : f32x4{-m_use[nt], -m_use[nt], -m_use[nt], -m_use[nt]});
        // (two head tiles: the query fragments from LDS, through an opaque lane index
        // that keeps the compiler from hoisting them back into registers)
        int ql = lane;
        if (NT > 1) asm volatile("" : "+v"(ql));
  #pragma unroll
        for (int s = 0; s < 4; ++s)
          S = mfma16x16x32(ka[s], NT == 1 ? qb[nt][s] : __builtin_bit_cast(bf16x8, qs[(nt * 4 + s) * 64 + ql]), S);
        if (KV8) {
  #pragma unroll
          for (int j = 0; j < 4; ++j) S[j] = fmaf(S[j], exp_scale(kexp, j), negm[nt][j]);
        }
        float lm = kNegInf;
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int krow = 4 * g + j;
          float x = S[j];
          if (PE == LAZYATTN_PE_ALIBI) x -= slope[nt] * static_cast<float>(pcol[nt] - (inf.start + krow));
          x = (krow < inf.len) ? x : kNegInf;
          S[j] = x;
          lm = fmaxf(lm, x);
        }
        // raise the reference only when a score outgrows it by 2^8 (exact:
        // numerator and denominator share it); the test is one compare and a ballot
        const bool want = (lm > kRescaleSlack) || (m_run[nt] == kNegInf && lm > kNegInf);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(want) != 0, 0)) {
          float pm = fmaxf(lm, __shfl_xor(lm, 16));
          pm = fmaxf(pm, __shfl_xor(pm, 32));
          const bool raise = (pm > kRescaleSlack) || (m_run[nt] == kNegInf && pm > kNegInf);
          const float m_new = raise ? m_use[nt] + pm : m_run[nt];
          const float mu_new = (m_new == kNegInf) ? 0.f : m_new;
          const float delta = mu_new - m_use[nt];
          const float alpha = (m_new == m_run[nt]) ? 1.f : __builtin_amdgcn_exp2f(m_run[nt] - m_new);
          S -= delta;
  #pragma unroll
          for (int dt = 0; dt < 8; ++dt) O[dt][nt] *= alpha;
          l_run[nt] *= alpha;
          m_run[nt] = m_new;
          m_use[nt] = mu_new;
          if (NT == 1) negm[nt] = f32x4{-mu_new, -mu_new, -mu_new, -mu_new};
        }
        float pe[4];
  #pragma unroll
        for (int j = 0; j < 4; ++j) pe[j] = __builtin_amdgcn_exp2f(S[j]);
        const uint32_t p01 = pack_bf16x2(pe[0], pe[1]), p23 = pack_bf16x2(pe[2], pe[3]);
        // row sum of the bf16-rounded weights that enter P.V
        l_run[nt] += (bf_lo(p01) + bf_hi(p01)) + (bf_lo(p23) + bf_hi(p23));
        s16x4 pb = __builtin_bit_cast(s16x4, make_uint2(p01, p23));
        if (KV8) {
          // each token's value scale goes on its weight (tokens past the entry's
          // length have weight 0 and codes zeroed above)
          pb = __builtin_bit_cast(s16x4, make_uint2(pack_bf16x2(pe[0] * exp_scale(vexp, 0), pe[1] * exp_scale(vexp, 1)),
                                                    pack_bf16x2(pe[2] * exp_scale(vexp, 2), pe[3] * exp_scale(vexp, 3))));
        }
  #pragma unroll
        for (int dt = 0; dt < 8; ++dt) O[dt][nt] = mfma16x16x16(__builtin_bit_cast(s16x4, v[dt]), pb, O[dt][nt]);
      }
  };

  // the wave's entries, nk of them from the staged table: kRing in flight
  auto run_ring = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int sl = 0; sl < kRing; ++sl) {
      fetch(curb[sl], frb[sl]);
      load_kv(curb[sl].blk, krb[sl], vrb[sl]);
      put_phase(sl, curb[sl].start);
    }
    // The slots run in order and the group loop has one exit, after the last
    // slot's refill: on every path into a slot's processing the other slots'
    // loads are the newer ones, so the wait for this slot's data leaves them in
    // flight.  A slot's phase row is rewritten only after its entry's reads of
    // it (the same wave's LDS operations complete in order).
    const int ngrp = nk / kRing;
    for (int it = 0; it < ngrp; ++it) {
#pragma unroll
      for (int sl = 0; sl < kRing; ++sl) {
        process(curb[sl], frb[sl], krb[sl], vrb[sl], sl);
        __builtin_amdgcn_sched_barrier(0);
        fetch(curb[sl], frb[sl]);
        load_kv(curb[sl].blk, krb[sl], vrb[sl]);
        put_phase(sl, curb[sl].start);
      }
    }
    const int rem = nk - ngrp * kRing;
#pragma unroll
    for (int sl = 0; sl + 1 < kRing; ++sl)
      if (rem > sl) process(curb[sl], frb[sl], krb[sl], vrb[sl], sl);
  };

  if (runs) {
    // ---- shared-run item: one wave, its entries in order, its own partials ----
    if (run_n == 0) return;
    for (int i = lane; i < run_n; i += 64) {
      // an item entry: block, key offset from the item's base (bits 58..32), length
      const uint64_t w = A.words[run_w0 + i];
      const uint32_t off = static_cast<uint32_t>(w >> 32) & 0x7ffffffu;
      tst[tab_base + i] = off;
      ten[tab_base + i] = off + static_cast<uint32_t>(w >> 59);
      tbk[tab_base + i] = static_cast<uint32_t>(w);
      if (PE == kPeFramed) tfr[tab_base + i] = 0;
    }
    // only this wave reads these rows: its own LDS writes are ordered before its reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    nk = run_n;
    kl = 0;
    run_ring();
    // column (occurrence j, head): o / l in fp16 and (m, l) to the occurrence's slot;
    // lane (g, n) holds channels 16 dt + 4 g .. + 3 of column n
    float lt = l_run[0] + __shfl_xor(l_run[0], 16);
    lt += __shfl_xor(lt, 32);
    if (n < Gw) {
      const int j = n / G;
      const size_t prow = static_cast<size_t>(run_ref0 + j) * Hq + kvh * G + (n - j * G);
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 o = O[dt][0];
        *reinterpret_cast<uint2*>(A.o_part + prow * kPD + 16 * dt + 4 * g) =
            make_uint2(pack_f16x2(o[0] * inv, o[1] * inv), pack_f16x2(o[2] * inv, o[3] * inv));
      }
      if (g == 0) *reinterpret_cast<float2*>(A.ml_part + prow * 2) = make_float2(m_run[0], lt);
    }
    return;
  }

  const int n_split = max(0, e_end - e_begin);
  for (int c0 = 0; c0 < n_split; c0 += kTab) {
    const int cn = min(kTab, n_split - c0);
    if (c0 > 0) __syncthreads();                     // every wave is done with the previous chunk
    for (int i = tid; i < cn; i += 256) {
      const int ei = e_begin + c0 + i;
      const uint64_t w = trow[ei];
      tst[i] = word_start(w);
      ten[i] = (ei + 1 < ne) ? reinterpret_cast<const uint32_t*>(trow + ei + 1)[1] : static_cast<uint32_t>(L);
      tbk[i] = word_block(w);
      if (PE == kPeFramed) tfr[i] = frow_v[ei];
    }
    __syncthreads();
    nk = max(0, (cn - wv + 3) >> 2);
    kl = 0;
    if (nk == 0) continue;
    run_ring();
  }

  // ---- merge the four waves ------------------------------------------------------
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = l_run[nt] + __shfl_xor(l_run[nt], 16);
    lt += __shfl_xor(lt, 32);
    l_run[nt] = lt;
    if (g == 0) {
      ml_s[(wave * NT * 16 + nt * 16 + n) * 2 + 0] = m_run[nt];
      ml_s[(wave * NT * 16 + nt * 16 + n) * 2 + 1] = lt;
    }
  }
  // one 16-column tile at a time through the [4][16][kOS] buffer
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    __syncthreads();
    const int col = nt * 16 + n;
    if (col < Gw) {
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_s[(w * NT * 16 + col) * 2]);
      const float f = (M == kNegInf || m_run[nt] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run[nt] - M);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4*>(o_s + (wave * 16 + n) * kOS + 16 * dt + 4 * g) = O[dt][nt] * f;
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * kPD; idx += 256) {
      const int c16 = idx / kPD, d = idx - c16 * kPD, col2 = nt * 16 + c16;
      if (col2 >= Gw) break;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_s[(w * NT * 16 + col2) * 2]);
      float lsum = 0.f, osum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = ml_s[(w * NT * 16 + col2) * 2];
        if (M != kNegInf && mw != kNegInf) lsum += __builtin_amdgcn_exp2f(mw - M) * ml_s[(w * NT * 16 + col2) * 2 + 1];
        osum += o_s[(w * 16 + c16) * kOS + d];
      }
      const int h = kvh * G + hb + col2;
      const size_t rowoff = static_cast<size_t>(r) * Hq + h;
      if (A.splits == 1) {
        const float val = lsum > 0.f ? osum / lsum : 0.f;
        A.out[rowoff * kPD + d] = static_cast<uint16_t>(pack_bf16x2(val, 0.f) & 0xffffu);
      } else {
        const size_t prow = static_cast<size_t>(split) * A.R * Hq + rowoff;
        A.o_part[prow * kPD + d] = static_cast<uint16_t>(pack_f16x2(lsum > 0.f ? osum / lsum : 0.f, 0.f) & 0xffffu);
        if (d == 0) *reinterpret_cast<float2*>(A.ml_part + prow * 2) = make_float2(M, lsum);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Materialise-then-attend baseline: per-request copies of the KV with K rows
// rotated at their absolute positions, and queries rotated at theirs, so a
// rotation-free kernel can attend over the copy.  Comparison only.
// One work-group per (entry, request, KV head): lane l of each wave rotates
// channel pair l of 4 key rows (phase R(t) stepped by R(1) per row); V is
// copied 16 B per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void materialize_kernel(const uint16_t* kpool, const uint16_t* vpool,
                                                          const uint64_t* src_tab, const uint64_t* dst_tab,
                                                          const int32_t* n_ent, int max_entries, int Hkv,
                                                          uint16_t* dk, uint16_t* dv, RopeRev rope) {
  const int e = blockIdx.x, r = blockIdx.y, h = blockIdx.z;
  if (e >= n_ent[r]) return;
  const uint64_t w = src_tab[static_cast<size_t>(r) * max_entries + e];
  const uint32_t src = word_block(w), dst = word_block(dst_tab[static_cast<size_t>(r) * max_entries + e]);
  const int start = static_cast<int>(word_start(w));
  const int tid = threadIdx.x, pair = tid & 63, row0 = 4 * (tid >> 6);
  const size_t sb = (static_cast<size_t>(src) * Hkv + h) * (kBlock * kPD);
  const size_t db = (static_cast<size_t>(dst) * Hkv + h) * (kBlock * kPD);
  const uint32_t* ks = reinterpret_cast<const uint32_t*>(kpool + sb) + pair;
  uint32_t* kd = reinterpret_cast<uint32_t*>(dk + db) + pair;
  float2 ph = unit_phase(start + row0, rope.rev[pair]);
  const float2 step = unit_phase(1, rope.rev[pair]);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = row0 + k;
    kd[row * (kPD / 2)] = rotate_pair(ks[row * (kPD / 2)], ph);
    ph = cmul(ph, step);
  }
  reinterpret_cast<uint4*>(dv + db)[tid] = reinterpret_cast<const uint4*>(vpool + sb)[tid];
}

// Keys turned once for the prefill (LAZYATTN_FLAG_KEYS_ONCE).  Wave w of
// work-group (x, r) takes entry e = 4 x + w of request r and writes every KV
// head's 16 key rows, each turned by R(t - c) (t its position, c = the
// request's first new position), to out[r][kvh][e] ([R][Hkv][max_entries]
// chunks of 16 x D: one request and KV head's keys are contiguous, in table
// order, as the attention kernel's work-groups read them).  Lane l moves 16 bytes of rows l / 16 + 4 i
// (i = 0..3), channels 8 (l % 16) .. + 7, i.e. four channel pairs: its 16
// phases are formed once per entry (angle reduced in double) and serve every
// head.  Rows past the entry's length are turned too; the attention kernel
// masks their scores.
__global__ __launch_bounds__(256) void turn_keys_kernel(const uint16_t* kpool, const uint64_t* tables,
                                                        const int32_t* n_ent, const int32_t* ctx,
                                                        const int32_t* cu_q, int max_entries, int Hkv,
                                                        uint16_t* out, RopeRev rope) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.y;
  const int e = 4 * static_cast<int>(blockIdx.x) + wave;
  if (e >= min(n_ent[r], max_entries)) return;
  const uint64_t w = tables[static_cast<size_t>(r) * max_entries + e];
  const int c = ctx[r] - (cu_q[r + 1] - cu_q[r]);
  const int n0 = static_cast<int>(word_start(w)) - c + (lane >> 4);
  const int j0 = 4 * (lane & 15);
  float2 ph[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) ph[i][q] = unit_phase_turns(n0 + 4 * i, rope.rev[j0 + q]);
  const int off = (lane >> 4) * kPD + 8 * (lane & 15);
  const uint16_t* src = kpool + static_cast<size_t>(word_block(w)) * Hkv * (kBlock * kPD) + off;
  uint16_t* dst = out + (static_cast<size_t>(r) * Hkv * max_entries + e) * (kBlock * kPD) + off;
#pragma unroll 2
  for (int kvh = 0; kvh < Hkv; ++kvh) {
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const uint4*>(src + kvh * (kBlock * kPD) + 4 * i * kPD);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 t = make_uint4(rotate_pair(v[i].x, ph[i][0]), rotate_pair(v[i].y, ph[i][1]),
                                 rotate_pair(v[i].z, ph[i][2]), rotate_pair(v[i].w, ph[i][3]));
      *reinterpret_cast<uint4*>(dst + static_cast<size_t>(kvh) * max_entries * (kBlock * kPD) + 4 * i * kPD) = t;
    }
  }
}

// One work-group per (query row of a request, request): lane l rotates
// channel pair l of every head of that token by R(p).
__global__ __launch_bounds__(64) void rotate_queries_kernel(const uint16_t* q, const int32_t* cu_q,
                                                            const int32_t* ctx, int Hq, uint16_t* q_out,
                                                            RopeRev rope) {
  const int j = blockIdx.x, r = blockIdx.y, lane = threadIdx.x;
  const int q0 = cu_q[r], q_len = cu_q[r + 1] - q0;
  if (j >= q_len) return;
  const int pos = ctx[r] - q_len + j;
  const float2 ph = unit_phase(pos, rope.rev[lane]);
  const size_t base = static_cast<size_t>(q0 + j) * Hq * kPD;
  for (int hh = 0; hh < Hq; ++hh) {
    const uint32_t x = reinterpret_cast<const uint32_t*>(q + base + static_cast<size_t>(hh) * kPD)[lane];
    reinterpret_cast<uint32_t*>(q_out + base + static_cast<size_t>(hh) * kPD)[lane] = rotate_pair(x, ph);
  }
}

// ---------------------------------------------------------------------------
// fp32 attention on the vector ALU, for the float32 dtype.  One wave per
// (query row, head); lane i owns channel pair i; keys are visited one by one
// with an online softmax.  Used for small fp32 cases (correctness path).
// ---------------------------------------------------------------------------
struct NaiveArgs {
  const float* q;
  const int32_t* cu_q;  // NULL: one query per request at row r (decode)
  const float* kpool;
  const float* vpool;
  const uint64_t* tables;
  const int32_t* n_ent;
  const int32_t* ctx;
  const float* alibi;
  float* out;
  int32_t Hq, Hkv, G, D, max_entries, pe;
  float scale;
  RopeRev rope;
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(64) void attn_f32_kernel(const NaiveArgs A) {
  const int j = blockIdx.x, r = blockIdx.y, h = blockIdx.z, i = threadIdx.x;
  const int qrow0 = A.cu_q ? A.cu_q[r] : r;
  const int q_len = A.cu_q ? A.cu_q[r + 1] - qrow0 : 1;
  if (j >= q_len) return;
  const int L = A.ctx[r], ne = A.n_ent[r];
  const int p = L - q_len + j;
  const int kvh = h / A.G, D = A.D;
  const bool act = 2 * i < D;
  const uint64_t* trow = A.tables + static_cast<size_t>(r) * A.max_entries;
  const float* qv = A.q + (static_cast<size_t>(qrow0 + j) * A.Hq + h) * D;
  const float q0 = act ? qv[2 * i] : 0.f, q1 = act ? qv[2 * i + 1] : 0.f;
  const double rev = (act && A.pe == LAZYATTN_PE_ROPE) ? A.rope.rev[i] : 0.0;
  const float slope = (A.pe == LAZYATTN_PE_ALIBI) ? alibi_slope(A.alibi, h, A.Hq) : 0.f;
  float m = kNegInf, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int e = 0; e < ne; ++e) {
    const EntryInfo inf = entry_info(trow, e, ne, L);
    if (inf.start > p) break;
    for (int rr = 0; rr < inf.len; ++rr) {
      const int t = inf.start + rr;
      if (t > p) break;
      const size_t kb = ((static_cast<size_t>(inf.blk) * A.Hkv + kvh) * kBlock + rr) * D;
      float k0 = act ? A.kpool[kb + 2 * i] : 0.f, k1 = act ? A.kpool[kb + 2 * i + 1] : 0.f;
      if (A.pe == LAZYATTN_PE_ROPE) {
        const float2 ph = unit_phase(t - p, rev);
        const float y0 = k0 * ph.x - k1 * ph.y, y1 = k0 * ph.y + k1 * ph.x;
        k0 = y0;
        k1 = y1;
      }
      float z = wave_sum(q0 * k0 + q1 * k1) * A.scale;
      if (A.pe == LAZYATTN_PE_ALIBI) z -= slope * static_cast<float>(p - t);
      const float m_new = fmaxf(m, z);
      const float alpha = expf(m - m_new);
      const float pz = expf(z - m_new);
      const size_t vb = (static_cast<size_t>(inf.blk) * A.Hkv + kvh) * static_cast<size_t>(D) * kBlock;
      const float v0 = act ? A.vpool[vb + (2 * i) * kBlock + rr] : 0.f;
      const float v1 = act ? A.vpool[vb + (2 * i + 1) * kBlock + rr] : 0.f;
      l = l * alpha + pz;
      o0 = o0 * alpha + pz * v0;
      o1 = o1 * alpha + pz * v1;
      m = m_new;
    }
  }
  if (act) {
    float* ov = A.out + (static_cast<size_t>(qrow0 + j) * A.Hq + h) * D;
    ov[2 * i] = o0 / l;
    ov[2 * i + 1] = o1 / l;
  }
}

// ---------------------------------------------------------------------------
// KV append: scatter new tokens' content-only K/V into pool slots.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void append_kv_kernel(T* kpool, T* vpool, const T* knew, const T* vnew, const int64_t* slots, int Hkv,
                                 int D) {
  const int i = blockIdx.x, h = blockIdx.y;
  const int64_t slot = slots[i];
  const int64_t blk = slot / kBlock;
  const int row = static_cast<int>(slot - blk * kBlock);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    const size_t src = (static_cast<size_t>(i) * Hkv + h) * D + d;
    kpool[((static_cast<size_t>(blk) * Hkv + h) * kBlock + row) * D + d] = knew[src];
    vpool[((static_cast<size_t>(blk) * Hkv + h) * D + d) * kBlock + row] = vnew[src];
  }
}

// KV append into a pool in document-local frames: the key is turned by
// R(frame_index) (its position within its frame) before it is stored; one
// thread per channel pair, the angle reduced in double as everywhere else.
__global__ void append_kv_framed_kernel(uint16_t* kpool, uint16_t* vpool, const uint16_t* knew, const uint16_t* vnew,
                                        const int64_t* slots, const int32_t* frame_index, int Hkv, int D,
                                        const RopeRev rope) {
  const int i = blockIdx.x, h = blockIdx.y;
  const int64_t slot = slots[i];
  const int64_t blk = slot / kBlock;
  const int row = static_cast<int>(slot - blk * kBlock);
  const int j = frame_index[i];
  const size_t src = (static_cast<size_t>(i) * Hkv + h) * D;
  const uint32_t* k2 = reinterpret_cast<const uint32_t*>(knew + src);
  uint32_t* kdst = reinterpret_cast<uint32_t*>(kpool + ((static_cast<size_t>(blk) * Hkv + h) * kBlock + row) * D);
  for (int pr = threadIdx.x; pr < D / 2; pr += blockDim.x) kdst[pr] = rotate_pair(k2[pr], unit_phase(j, rope.rev[pr]));
  for (int d = threadIdx.x; d < D; d += blockDim.x)
    vpool[((static_cast<size_t>(blk) * Hkv + h) * D + d) * kBlock + row] = vnew[src + d];
}

// FP8 append: each new K row and V row (128 values of one token and head) is
// quantised whole.  Exponent e = the smallest with max|x| <= 448 * 2^e (at
// least -127; 0 for an all-zero row); code = x * 2^-e rounded to the nearest
// e4m3 value, ties to even, saturated at 448; the sign is kept (also of zero).
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7eu;
  } else if (a < 0.015625f) {                     // below 2^-6: steps of 2^-9 (8 = smallest normal)
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    const int E = __builtin_amdgcn_frexp_expf(a) - 1;                  // a in [2^E, 2^(E+1))
    const int m = static_cast<int>(__builtin_rintf(__builtin_amdgcn_ldexpf(a, 3 - E)));   // 8..16
    code = static_cast<uint32_t>((E + 7) * 8 + (m - 8));              // m = 16 carries into the exponent
  }
  return sign | code;
}

__device__ __forceinline__ int fp8_row_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int Ea = __builtin_amdgcn_frexp_expf(amax) - 1;               // amax in [2^Ea, 2^(Ea+1))
  if (Ea - 7 <= -127) return -127;
  return (amax <= __builtin_amdgcn_ldexpf(1.75f, Ea)) ? Ea - 8 : Ea - 7;   // 448 = 1.75 * 2^8
}

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// One wave per (token, KV head); lane l holds channels 2l, 2l+1.  With
// frame_index (a pool in document-local frames) the key is first turned by
// R(frame_index[i]) in float, then quantised.
__global__ __launch_bounds__(64) void append_kv_fp8_kernel(uint8_t* kpool, uint8_t* vpool, const uint16_t* knew,
                                                           const uint16_t* vnew, const int64_t* slots,
                                                           const int32_t* frame_index, int Hkv, const RopeRev rope) {
  const int i = blockIdx.x, h = blockIdx.y, l = threadIdx.x;
  const int64_t slot = slots[i];
  const int64_t blk = slot / kBlock;
  const int row = static_cast<int>(slot - blk * kBlock);
  const size_t src = (static_cast<size_t>(i) * Hkv + h) * kPD;
  const uint32_t kw = reinterpret_cast<const uint32_t*>(knew + src)[l];
  const uint32_t vw = reinterpret_cast<const uint32_t*>(vnew + src)[l];
  float k0 = bf_lo(kw), k1 = bf_hi(kw);
  if (frame_index) {
    const float2 ph = unit_phase(frame_index[i], rope.rev[l]);
    const float y0 = k0 * ph.x - k1 * ph.y, y1 = k0 * ph.y + k1 * ph.x;
    k0 = y0;
    k1 = y1;
  }
  const float v0 = bf_lo(vw), v1 = bf_hi(vw);
  const int ek = fp8_row_exponent(wave_max64(fmaxf(fabsf(k0), fabsf(k1))));
  const int ev = fp8_row_exponent(wave_max64(fmaxf(fabsf(v0), fabsf(v1))));
  const size_t chunk = (static_cast<size_t>(blk) * Hkv + h) * kChunk8;
  uint8_t* kc = kpool + chunk;
  uint8_t* vc = vpool + chunk;
  const uint32_t c0 = f32_to_e4m3(__builtin_amdgcn_ldexpf(k0, -ek));
  const uint32_t c1 = f32_to_e4m3(__builtin_amdgcn_ldexpf(k1, -ek));
  reinterpret_cast<uint16_t*>(kc + row * kPD)[l] = static_cast<uint16_t>(c0 | (c1 << 8));
  vc[(2 * l) * kBlock + row] = static_cast<uint8_t>(f32_to_e4m3(__builtin_amdgcn_ldexpf(v0, -ev)));
  vc[(2 * l + 1) * kBlock + row] = static_cast<uint8_t>(f32_to_e4m3(__builtin_amdgcn_ldexpf(v1, -ev)));
  if (l == 0) {
    kc[16 * kPD + row] = static_cast<uint8_t>(static_cast<int8_t>(ek));
    vc[16 * kPD + row] = static_cast<uint8_t>(static_cast<int8_t>(ev));
  }
}

// ---------------------------------------------------------------------------
// Table decode, exactly as the attention kernels see it.
// ---------------------------------------------------------------------------
__global__ void debug_decode_kernel(const uint64_t* tables, const int32_t* n_ent, const int32_t* ctx, int E,
                                    int32_t* out) {
  const int r = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int ne = n_ent[r];
  int32_t* o = out + (static_cast<size_t>(r) * E + e) * 3;
  if (e < ne) {
    const EntryInfo inf = entry_info(tables + static_cast<size_t>(r) * E, e, ne, ctx[r]);
    o[0] = static_cast<int32_t>(inf.blk);
    o[1] = inf.start;
    o[2] = inf.len;
  } else {
    o[0] = o[1] = o[2] = -1;
  }
}

// ---------------------------------------------------------------------------
// host launch helpers
// ---------------------------------------------------------------------------
static lazyattn_status launched() {
  return hipGetLastError() == hipSuccess ? LAZYATTN_OK : LAZYATTN_EHIP;
}

static lazyattn_status check_batch(const lazyattn_batch* b) {
  if (!b || b->num_reqs < 0) return LAZYATTN_EINVAL;
  if (b->num_reqs > 0) {
    if (!b->block_tables || !b->num_entries || !b->ctx_lens) return LAZYATTN_EINVAL;
    if (b->max_entries < 1) return LAZYATTN_EINVAL;
  }
  return LAZYATTN_OK;
}

// Decode work-groups reserve at least this much LDS, so that at most two share
// a CU (160 KiB each) whatever the positional encoding: with three, the
// concurrent streams thrash the L2 that shared document blocks are reused from
// (measured slower on the Llama-3.1-8B decode), and the rotation-free control
// keeps the occupancy of the RoPE kernel it is compared with.
constexpr size_t kDecodeLdsFloor = 56 * 1024;

static size_t decode_lds_bytes(int nt) {
  const size_t need = (4 * kRing * 64 * 2 + 4 * static_cast<size_t>(nt) * 16 * 2 + 4 * 16 * kOS + 16 * 64 * 2 +
                       (nt > 1 ? static_cast<size_t>(nt) * 4 * 64 * 4 : 0)) *
                      sizeof(float);
  return need > kDecodeLdsFloor ? need : kDecodeLdsFloor;
}

// ---------------------------------------------------------------------------
// launchers (host)
// ---------------------------------------------------------------------------

static lazyattn_status merge_launch(int rows_total, int splits, const void* workspace, void* out, hipStream_t stream) {
  const uint16_t* o_part = static_cast<const uint16_t*>(workspace);
  const float* ml_part = reinterpret_cast<const float*>(o_part + static_cast<size_t>(splits) * rows_total * kPD);
  if (splits > 4)
    hipLaunchKernelGGL(merge_kernel<16>, dim3((rows_total + 15) / 16), dim3(256), 0, stream, o_part, ml_part,
                       static_cast<uint16_t*>(out), rows_total, splits, nullptr, nullptr, 0);
  else
    hipLaunchKernelGGL(merge_kernel<4>, dim3((rows_total + 15) / 16), dim3(256), 0, stream, o_part, ml_part,
                       static_cast<uint16_t*>(out), rows_total, splits, nullptr, nullptr, 0);
  return launched();
}

// Whether the prefill groups the query tiles of a (split, request, KV head)
// unit per XCD: units of at least 32 tiles, U units a multiple of 8, or U
// dividing 8 with the tiles divisible by 8 / U
static bool xcd_grouping(long long n_qt, long long U) {
  if (n_qt < 32 || U < 1) return false;
  if (U % 8 == 0) return true;
  return 8 % U == 0 && n_qt % (8 / U) == 0;
}

// Validates and launches the prefill attention kernel; *splits_out = splits used.
static lazyattn_status prefill_attend(const lazyattn_config* cfg, const void* q, const int32_t* cu_q_lens,
                                      int32_t total_q, int32_t max_q_len, const void* k_pool, const void* v_pool,
                                      int64_t num_blocks, const lazyattn_batch* batch, int32_t num_splits, void* out,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream, int* splits_out) {
  *splits_out = 1;
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if ((st = check_batch(batch)) != LAZYATTN_OK) return st;
  if (total_q < 0 || max_q_len < 0 || num_splits < 0 || num_splits > 64 || num_blocks < 0) return LAZYATTN_EINVAL;
  if (batch->num_reqs == 0 || total_q == 0) return LAZYATTN_OK;
  if (!q || !cu_q_lens || !k_pool || !v_pool || !out || num_blocks < 1 || max_q_len < 1) return LAZYATTN_EINVAL;
  const int R = batch->num_reqs, Hq = cfg->num_q_heads, Hkv = cfg->num_kv_heads, G = Hq / Hkv;
  const RopeRev rope = make_rope_rev(cfg);
  const float scale = softmax_scale_of(cfg);

  const bool framed = batch->frame_starts != nullptr;
  const bool fp8 = cfg->kv_format == LAZYATTN_KV_FP8_E4M3;
  if (framed && (cfg->dtype != LAZYATTN_BF16 || cfg->pe != LAZYATTN_PE_ROPE)) return LAZYATTN_EUNSUPPORTED;
  if (cfg->dtype == LAZYATTN_F32) {
    if (max_q_len > 0x7fffffff || R > 65535 || Hq > 65535) return LAZYATTN_EUNSUPPORTED;
    NaiveArgs a{static_cast<const float*>(q), cu_q_lens, static_cast<const float*>(k_pool),
                static_cast<const float*>(v_pool), batch->block_tables, batch->num_entries, batch->ctx_lens,
                cfg->alibi_slopes, static_cast<float*>(out), Hq, Hkv, G, cfg->head_dim, batch->max_entries,
                cfg->pe, scale, rope};
    hipLaunchKernelGGL(attn_f32_kernel, dim3(max_q_len, R, Hq), dim3(64), 0, stream, a);
    return launched();
  }

  if (G > 256) return LAZYATTN_EUNSUPPORTED;
  const int splits = num_splits > 0 ? num_splits : choose_prefill_splits(cfg, R, max_q_len, batch->max_entries);
  // keys turned once (plain content-only pool, RoPE): after the partials in the workspace
  const bool once = !framed && !fp8 && prefill_keys_once(cfg, max_q_len);
  const size_t part_bytes = prefill_partials_bytes(cfg, total_q, splits);
  const size_t need = once ? prefill_turned_keys_offset(part_bytes) +
                                 prefill_turned_keys_bytes(cfg, R, batch->max_entries)
                           : part_bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return LAZYATTN_EWORKSPACE;
  const int m_q = prefill_positions_per_tile(G);
  const long long n_qt = (max_q_len + m_q - 1) / m_q;
  const long long gx = n_qt * splits;
  if (R > 65535 || Hkv > 65535 || gx > 0x7fffffff) return LAZYATTN_EUNSUPPORTED;
  uint16_t* o_part = splits > 1 ? static_cast<uint16_t*>(workspace) : nullptr;
  float* ml_part = splits > 1 ? reinterpret_cast<float*>(o_part + static_cast<size_t>(splits) * total_q * Hq * kPD)
                              : nullptr;
  PrefillArgs a{static_cast<const uint16_t*>(q), cu_q_lens, static_cast<const uint16_t*>(k_pool),
                static_cast<const uint16_t*>(v_pool), batch->block_tables, batch->num_entries, batch->ctx_lens,
                batch->frame_starts, batch->req_order, cfg->alibi_slopes, static_cast<uint16_t*>(out), o_part,
                ml_part,
                once ? reinterpret_cast<const uint16_t*>(static_cast<const char*>(workspace) +
                                                         prefill_turned_keys_offset(part_bytes))
                     : nullptr,
                Hq, Hkv, G, batch->max_entries, total_q, m_q,
                prefill_entries_per_split(batch->max_entries, splits), splits, static_cast<int32_t>(n_qt),
                xcd_grouping(n_qt, static_cast<long long>(splits) * R * Hkv) ? 1 : 0,
                (cfg->flags & LAZYATTN_FLAG_EXACT_MAX) ? 1 : 0, scale * kLog2e, rope};
  const dim3 grid(static_cast<unsigned>(gx), R, static_cast<unsigned>(Hkv));
  const dim3 block(kPrefillThreads);
  if (once) {
    hipLaunchKernelGGL(turn_keys_kernel, dim3((batch->max_entries + 3) / 4, R), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(k_pool), batch->block_tables, batch->num_entries,
                       batch->ctx_lens, cu_q_lens, batch->max_entries, Hkv, const_cast<uint16_t*>(a.kturned), rope);
    if ((st = launched()) != LAZYATTN_OK) return st;
    hipLaunchKernelGGL((prefill_bf16_kernel<kPeKeysTurned, 0>), grid, block, 0, stream, a);
  } else if (fp8) {
    switch (framed ? kPeFramed : cfg->pe) {
      case kPeFramed: hipLaunchKernelGGL((prefill_bf16_kernel<kPeFramed, 1>), grid, block, 0, stream, a); break;
      case LAZYATTN_PE_ROPE: hipLaunchKernelGGL((prefill_bf16_kernel<LAZYATTN_PE_ROPE, 1>), grid, block, 0, stream, a); break;
      case LAZYATTN_PE_NONE: hipLaunchKernelGGL((prefill_bf16_kernel<LAZYATTN_PE_NONE, 1>), grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL((prefill_bf16_kernel<LAZYATTN_PE_ALIBI, 1>), grid, block, 0, stream, a); break;
    }
  } else {
    switch (framed ? kPeFramed : cfg->pe) {
      case kPeFramed: hipLaunchKernelGGL((prefill_bf16_kernel<kPeFramed, 0>), grid, block, 0, stream, a); break;
      case LAZYATTN_PE_ROPE: hipLaunchKernelGGL((prefill_bf16_kernel<LAZYATTN_PE_ROPE, 0>), grid, block, 0, stream, a); break;
      case LAZYATTN_PE_NONE: hipLaunchKernelGGL((prefill_bf16_kernel<LAZYATTN_PE_NONE, 0>), grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL((prefill_bf16_kernel<LAZYATTN_PE_ALIBI, 0>), grid, block, 0, stream, a); break;
    }
  }
  *splits_out = splits;
  return launched();
}

template <int PEV, int NTV, int KV8, int RUNS>
static void launch_decode_one(dim3 grid, size_t lds, hipStream_t stream, const DecodeArgs& a) {
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_bf16_kernel<PEV, NTV, KV8, RUNS>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  hipLaunchKernelGGL((decode_bf16_kernel<PEV, NTV, KV8, RUNS>), grid, dim3(256), lds, stream, a);
}

// Groups of 17..32 heads over a plain bf16 content-only pool: one wave holds
// all of them (two 16-column tiles), so every block is read and turned once
static void launch_decode_wide(int pe_sel, dim3 grid, size_t lds, hipStream_t stream, const DecodeArgs& a) {
  switch (pe_sel) {
    case LAZYATTN_PE_ROPE: launch_decode_one<LAZYATTN_PE_ROPE, 2, 0, 0>(grid, lds, stream, a); break;
    case LAZYATTN_PE_NONE: launch_decode_one<LAZYATTN_PE_NONE, 2, 0, 0>(grid, lds, stream, a); break;
    default: launch_decode_one<LAZYATTN_PE_ALIBI, 2, 0, 0>(grid, lds, stream, a); break;
  }
}

// RUNS: the shared-run decode (a content-only pool: no framed instantiation)
template <int KV8, int RUNS>
static void launch_decode(int pe_sel, dim3 grid, size_t lds, hipStream_t stream, const DecodeArgs& a) {
  switch (pe_sel) {
    case kPeFramed:
      if (!RUNS) launch_decode_one<kPeFramed, 1, KV8, 0>(grid, lds, stream, a);
      break;
    case LAZYATTN_PE_ROPE: launch_decode_one<LAZYATTN_PE_ROPE, 1, KV8, RUNS>(grid, lds, stream, a); break;
    case LAZYATTN_PE_NONE: launch_decode_one<LAZYATTN_PE_NONE, 1, KV8, RUNS>(grid, lds, stream, a); break;
    default: launch_decode_one<LAZYATTN_PE_ALIBI, 1, KV8, RUNS>(grid, lds, stream, a); break;
  }
}

static lazyattn_status decode_attend(const lazyattn_config* cfg, const void* q, const void* k_pool,
                                     const void* v_pool, int64_t num_blocks, const lazyattn_batch* batch,
                                     int32_t num_splits, void* out, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream, int* splits_out) {
  *splits_out = 1;
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if ((st = check_batch(batch)) != LAZYATTN_OK) return st;
  if (num_splits < 0 || num_splits > 256 || num_blocks < 0) return LAZYATTN_EINVAL;
  if (batch->num_reqs == 0) return LAZYATTN_OK;
  if (!q || !k_pool || !v_pool || !out || num_blocks < 1) return LAZYATTN_EINVAL;
  const int R = batch->num_reqs, Hq = cfg->num_q_heads, Hkv = cfg->num_kv_heads, G = Hq / Hkv;
  const RopeRev rope = make_rope_rev(cfg);
  const float scale = softmax_scale_of(cfg);

  const bool framed = batch->frame_starts != nullptr;
  if (framed && (cfg->dtype != LAZYATTN_BF16 || cfg->pe != LAZYATTN_PE_ROPE)) return LAZYATTN_EUNSUPPORTED;
  if (cfg->dtype == LAZYATTN_F32) {
    if (R > 65535 || Hq > 65535) return LAZYATTN_EUNSUPPORTED;
    NaiveArgs a{static_cast<const float*>(q), nullptr, static_cast<const float*>(k_pool),
                static_cast<const float*>(v_pool), batch->block_tables, batch->num_entries, batch->ctx_lens,
                cfg->alibi_slopes, static_cast<float*>(out), Hq, Hkv, G, cfg->head_dim, batch->max_entries,
                cfg->pe, scale, rope};
    hipLaunchKernelGGL(attn_f32_kernel, dim3(1, R, Hq), dim3(64), 0, stream, a);
    return launched();
  }

  if (G > 32) return LAZYATTN_EUNSUPPORTED;
  const int splits = num_splits > 0 ? num_splits : choose_decode_splits(cfg, R, batch->max_entries);
  const size_t need = lazyattn_decode_workspace_size(cfg, R, batch->max_entries, splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return LAZYATTN_EWORKSPACE;
  if (R > 65535 || Hkv > 65535) return LAZYATTN_EUNSUPPORTED;
  uint16_t* o_part = splits > 1 ? static_cast<uint16_t*>(workspace) : nullptr;
  float* ml_part = splits > 1 ? reinterpret_cast<float*>(o_part + static_cast<size_t>(splits) * R * Hq * kPD) : nullptr;
  DecodeArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_pool),
               static_cast<const uint16_t*>(v_pool), batch->block_tables, batch->num_entries, batch->ctx_lens,
               batch->frame_starts, batch->req_order, cfg->alibi_slopes, static_cast<uint16_t*>(out), o_part,
               ml_part, R, Hq, Hkv, G, batch->max_entries, decode_entries_per_split(batch->max_entries, splits),
               splits, 1, scale * kLog2e, rope};
  // groups of 17..32 heads: one wave of two head tiles (plain bf16 content-only
  // pool), else two work-groups of 16 heads
  const bool wide = G > 16 && !framed && cfg->kv_format == LAZYATTN_KV_PLAIN;
  a.halves = (G > 16 && !wide) ? 2 : 1;
  dim3 grid(splits, Hkv, R);
  if (a.halves == 2) {
    const long long items = static_cast<long long>(splits) * Hkv * R;
    if ((items + 7) / 8 * 16 > 0x7fffffffLL) return LAZYATTN_EUNSUPPORTED;
    grid = dim3(static_cast<unsigned>((items + 7) / 8 * 16), 1, 1);
  }
  const size_t lds = decode_lds_bytes(wide ? 2 : 1);
  const int pe_sel = framed ? kPeFramed : cfg->pe;
  if (wide)
    launch_decode_wide(pe_sel, grid, lds, stream, a);
  else if (cfg->kv_format == LAZYATTN_KV_FP8_E4M3)
    launch_decode<1, 0>(pe_sel, grid, lds, stream, a);
  else
    launch_decode<0, 0>(pe_sel, grid, lds, stream, a);
  *splits_out = splits;
  return launched();
}

// ---------------------------------------------------------------------------
// Allocation-free decode (lazyattn_decode_noalloc): the split partials go to a
// device array owned by the library instead of a caller's workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory, so its device
// address is looked up once per device and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[LAZYATTN_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on its first use there).
static lazyattn_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LAZYATTN_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LAZYATTN_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LAZYATTN_OK;
}

}  // namespace lazyattn

using namespace lazyattn;

extern "C" {

lazyattn_status lazyattn_prefill_attend(const lazyattn_config* cfg, const void* q, const int32_t* cu_q_lens,
                                        int32_t total_q, int32_t max_q_len, const void* k_pool, const void* v_pool,
                                        int64_t num_blocks, const lazyattn_batch* batch, int32_t num_splits,
                                        void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int splits;
  return prefill_attend(cfg, q, cu_q_lens, total_q, max_q_len, k_pool, v_pool, num_blocks, batch, num_splits, out,
                        workspace, workspace_bytes, stream, &splits);
}

lazyattn_status lazyattn_prefill(const lazyattn_config* cfg, const void* q, const int32_t* cu_q_lens,
                                 int32_t total_q, int32_t max_q_len, const void* k_pool, const void* v_pool,
                                 int64_t num_blocks, const lazyattn_batch* batch, int32_t num_splits, void* out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int splits;
  lazyattn_status st = prefill_attend(cfg, q, cu_q_lens, total_q, max_q_len, k_pool, v_pool, num_blocks, batch,
                                      num_splits, out, workspace, workspace_bytes, stream, &splits);
  if (st != LAZYATTN_OK || splits <= 1) return st;
  return merge_launch(total_q * cfg->num_q_heads, splits, workspace, out, stream);
}

lazyattn_status lazyattn_decode_attend(const lazyattn_config* cfg, const void* q, const void* k_pool,
                                       const void* v_pool, int64_t num_blocks, const lazyattn_batch* batch,
                                       int32_t num_splits, void* out, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  int splits;
  return decode_attend(cfg, q, k_pool, v_pool, num_blocks, batch, num_splits, out, workspace, workspace_bytes,
                       stream, &splits);
}

lazyattn_status lazyattn_decode(const lazyattn_config* cfg, const void* q, const void* k_pool, const void* v_pool,
                                int64_t num_blocks, const lazyattn_batch* batch, int32_t num_splits, void* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int splits;
  lazyattn_status st = decode_attend(cfg, q, k_pool, v_pool, num_blocks, batch, num_splits, out, workspace,
                                     workspace_bytes, stream, &splits);
  if (st != LAZYATTN_OK || splits <= 1) return st;
  return merge_launch(batch->num_reqs * cfg->num_q_heads, splits, workspace, out, stream);
}

lazyattn_status lazyattn_decode_runs(const lazyattn_config* cfg, const void* q, const void* k_pool,
                                     const void* v_pool, int64_t num_blocks, int32_t num_reqs,
                                     const lazyattn_run_plan* plan, void* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if (!plan || num_reqs < 0 || num_blocks < 0 || plan->num_items < 0 || plan->num_words < 0 || plan->num_refs < 0)
    return LAZYATTN_EINVAL;
  const int Hq = cfg->num_q_heads, Hkv = cfg->num_kv_heads, G = Hq / Hkv;
  if (cfg->dtype != LAZYATTN_BF16 || G > 16) return LAZYATTN_EUNSUPPORTED;
  if (num_reqs == 0) return LAZYATTN_OK;
  if (!q || !k_pool || !v_pool || !out || num_blocks < 1 || !plan->req_ref_begin || plan->num_items % 32 != 0)
    return LAZYATTN_EINVAL;
  if (plan->num_items > 0 && (!plan->items || !plan->words || !plan->refs || !plan->req_refs))
    return LAZYATTN_EINVAL;
  const size_t need = lazyattn_decode_runs_workspace_size(cfg, plan->num_refs);
  if (need > 0 && (!workspace || workspace_bytes < need)) return LAZYATTN_EWORKSPACE;
  if (Hkv > 65535 || static_cast<long long>(num_reqs) * Hq > 0x7fffffffLL - 15) return LAZYATTN_EUNSUPPORTED;
  uint16_t* o_part = static_cast<uint16_t*>(workspace);
  float* ml_part = reinterpret_cast<float*>(o_part + static_cast<size_t>(plan->num_refs) * Hq * kPD);
  if (plan->num_items > 0) {
    // the per-request arrays are not read for a shared-run item; valid device
    // pointers stand in for them all the same
    DecodeArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_pool),
                 static_cast<const uint16_t*>(v_pool), reinterpret_cast<const uint64_t*>(plan->items),
                 plan->req_ref_begin, plan->req_ref_begin, nullptr, nullptr, cfg->alibi_slopes,
                 static_cast<uint16_t*>(out),
                 o_part, ml_part, num_reqs, Hq, Hkv, G, 1, 1, 1, 1, softmax_scale_of(cfg) * kLog2e,
                 make_rope_rev(cfg), plan->items, plan->words, plan->refs};
    const dim3 grid(static_cast<unsigned>(plan->num_items / 4), static_cast<unsigned>(Hkv));
    if (cfg->kv_format == LAZYATTN_KV_FP8_E4M3)
      launch_decode<1, 1>(cfg->pe, grid, decode_lds_bytes(1), stream, a);
    else
      launch_decode<0, 1>(cfg->pe, grid, decode_lds_bytes(1), stream, a);
    if ((st = launched()) != LAZYATTN_OK) return st;
  }
  const int rows_total = num_reqs * Hq;
  hipLaunchKernelGGL(merge_kernel<16>, dim3((rows_total + 15) / 16), dim3(256), 0, stream, o_part, ml_part,
                     static_cast<uint16_t*>(out), rows_total, 0, plan->req_ref_begin, plan->req_refs, Hq);
  return launched();
}

lazyattn_status lazyattn_decode_noalloc(const lazyattn_config* cfg, const void* q, const void* k_pool,
                                        const void* v_pool, int64_t num_blocks, const lazyattn_batch* batch,
                                        int32_t num_splits, void* out, hipStream_t stream) {
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if ((st = check_batch(batch)) != LAZYATTN_OK) return st;
  if (num_splits < 0 || num_splits > 256) return LAZYATTN_EINVAL;
  if (batch->num_reqs == 0) return LAZYATTN_OK;
  const size_t need = lazyattn_decode_workspace_size(cfg, batch->num_reqs, batch->max_entries, num_splits);
  if (need > LAZYATTN_DECODE_SCRATCH_BYTES) return LAZYATTN_EWORKSPACE;
  void* ws = nullptr;
  if (need > 0 && (st = scratch_of_current_device(&ws)) != LAZYATTN_OK) return st;
  return lazyattn_decode(cfg, q, k_pool, v_pool, num_blocks, batch, num_splits, out, ws,
                         need > 0 ? static_cast<size_t>(LAZYATTN_DECODE_SCRATCH_BYTES) : 0, stream);
}

lazyattn_status lazyattn_merge_splits(const lazyattn_config* cfg, int32_t num_rows, int32_t num_splits,
                                      const void* workspace, size_t workspace_bytes, void* out, hipStream_t stream) {
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if (num_rows < 0 || num_splits < 1 || num_splits > 256) return LAZYATTN_EINVAL;
  if (num_splits == 1 || num_rows == 0) return LAZYATTN_OK;
  if (cfg->dtype != LAZYATTN_BF16) return LAZYATTN_EUNSUPPORTED;
  if (!workspace || !out) return LAZYATTN_EINVAL;
  const long long rows_total = static_cast<long long>(num_rows) * cfg->num_q_heads;
  const size_t need = static_cast<size_t>(num_splits) * rows_total * (kPD * sizeof(uint16_t) + 2 * sizeof(float));
  if (workspace_bytes < need) return LAZYATTN_EWORKSPACE;
  if (rows_total > 0x7fffffffLL - 8) return LAZYATTN_EUNSUPPORTED;
  return merge_launch(static_cast<int>(rows_total), num_splits, workspace, out, stream);
}

lazyattn_status lazyattn_append_kv(const lazyattn_config* cfg, void* k_pool, void* v_pool, int64_t num_blocks,
                                   const void* k_new, const void* v_new, const int64_t* slots, int32_t n,
                                   hipStream_t stream) {
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if (n < 0 || num_blocks < 0) return LAZYATTN_EINVAL;
  if (n == 0) return LAZYATTN_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slots || num_blocks < 1) return LAZYATTN_EINVAL;
  if (cfg->num_kv_heads > 65535) return LAZYATTN_EUNSUPPORTED;
  const dim3 grid(n, cfg->num_kv_heads);
  if (cfg->kv_format == LAZYATTN_KV_FP8_E4M3) {
    hipLaunchKernelGGL(append_kv_fp8_kernel, grid, dim3(64), 0, stream, static_cast<uint8_t*>(k_pool),
                       static_cast<uint8_t*>(v_pool), static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), slots, nullptr, cfg->num_kv_heads, make_rope_rev(cfg));
  } else if (cfg->dtype == LAZYATTN_BF16) {
    hipLaunchKernelGGL(append_kv_kernel<uint16_t>, grid, dim3(128), 0, stream, static_cast<uint16_t*>(k_pool),
                       static_cast<uint16_t*>(v_pool), static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), slots, cfg->num_kv_heads, cfg->head_dim);
  } else {
    hipLaunchKernelGGL(append_kv_kernel<float>, grid, dim3(128), 0, stream, static_cast<float*>(k_pool),
                       static_cast<float*>(v_pool), static_cast<const float*>(k_new),
                       static_cast<const float*>(v_new), slots, cfg->num_kv_heads, cfg->head_dim);
  }
  return launched();
}

lazyattn_status lazyattn_append_kv_framed(const lazyattn_config* cfg, void* k_pool, void* v_pool, int64_t num_blocks,
                                          const void* k_new, const void* v_new, const int64_t* slots,
                                          const int32_t* frame_index, int32_t n, hipStream_t stream) {
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if (cfg->dtype != LAZYATTN_BF16 || cfg->pe != LAZYATTN_PE_ROPE) return LAZYATTN_EUNSUPPORTED;
  if (n < 0 || num_blocks < 0) return LAZYATTN_EINVAL;
  if (n == 0) return LAZYATTN_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slots || !frame_index || num_blocks < 1) return LAZYATTN_EINVAL;
  if (cfg->num_kv_heads > 65535) return LAZYATTN_EUNSUPPORTED;
  if (cfg->kv_format == LAZYATTN_KV_FP8_E4M3) {
    hipLaunchKernelGGL(append_kv_fp8_kernel, dim3(n, cfg->num_kv_heads), dim3(64), 0, stream,
                       static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), slots, frame_index,
                       cfg->num_kv_heads, make_rope_rev(cfg));
    return launched();
  }
  hipLaunchKernelGGL(append_kv_framed_kernel, dim3(n, cfg->num_kv_heads), dim3(64), 0, stream,
                     static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), slots, frame_index,
                     cfg->num_kv_heads, cfg->head_dim, make_rope_rev(cfg));
  return launched();
}

lazyattn_status lazyattn_materialize_kv(const lazyattn_config* cfg, const void* k_pool, const void* v_pool,
                                        int64_t num_blocks, const lazyattn_batch* batch,
                                        const uint64_t* dst_tables, void* dst_k_pool, void* dst_v_pool,
                                        int64_t dst_num_blocks, hipStream_t stream) {
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if ((st = check_batch(batch)) != LAZYATTN_OK) return st;
  if (cfg->dtype != LAZYATTN_BF16 || cfg->pe != LAZYATTN_PE_ROPE) return LAZYATTN_EUNSUPPORTED;
  if (batch->frame_starts) return LAZYATTN_EUNSUPPORTED;     // copies are made from a content-only pool
  if (cfg->kv_format != LAZYATTN_KV_PLAIN) return LAZYATTN_EUNSUPPORTED;
  if (batch->num_reqs == 0 || batch->max_entries == 0) return LAZYATTN_OK;
  if (!k_pool || !v_pool || !dst_tables || !dst_k_pool || !dst_v_pool || num_blocks < 1 || dst_num_blocks < 1)
    return LAZYATTN_EINVAL;
  if (batch->num_reqs > 65535 || cfg->num_kv_heads > 65535) return LAZYATTN_EUNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(batch->max_entries), batch->num_reqs, cfg->num_kv_heads);
  hipLaunchKernelGGL(materialize_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(k_pool),
                     static_cast<const uint16_t*>(v_pool), batch->block_tables, dst_tables, batch->num_entries,
                     batch->max_entries, cfg->num_kv_heads, static_cast<uint16_t*>(dst_k_pool),
                     static_cast<uint16_t*>(dst_v_pool), make_rope_rev(cfg));
  return launched();
}

lazyattn_status lazyattn_rotate_queries(const lazyattn_config* cfg, const void* q, const int32_t* cu_q_lens,
                                        int32_t total_q, int32_t max_q_len, const lazyattn_batch* batch,
                                        void* q_out, hipStream_t stream) {
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if ((st = check_batch(batch)) != LAZYATTN_OK) return st;
  if (cfg->dtype != LAZYATTN_BF16 || cfg->pe != LAZYATTN_PE_ROPE) return LAZYATTN_EUNSUPPORTED;
  if (total_q < 0 || max_q_len < 0) return LAZYATTN_EINVAL;
  if (batch->num_reqs == 0 || total_q == 0 || max_q_len == 0) return LAZYATTN_OK;
  if (!q || !cu_q_lens || !q_out) return LAZYATTN_EINVAL;
  if (batch->num_reqs > 65535) return LAZYATTN_EUNSUPPORTED;
  hipLaunchKernelGGL(rotate_queries_kernel, dim3(max_q_len, batch->num_reqs), dim3(64), 0, stream,
                     static_cast<const uint16_t*>(q), cu_q_lens, batch->ctx_lens, cfg->num_q_heads,
                     static_cast<uint16_t*>(q_out), make_rope_rev(cfg));
  return launched();
}

lazyattn_status lazyattn_debug_decode_tables(const lazyattn_batch* batch, int32_t* out, hipStream_t stream) {
  lazyattn_status st = check_batch(batch);
  if (st != LAZYATTN_OK) return st;
  if (batch->num_reqs == 0) return LAZYATTN_OK;
  if (!out) return LAZYATTN_EINVAL;
  if (batch->num_reqs > 65535) return LAZYATTN_EUNSUPPORTED;
  const int E = batch->max_entries;
  hipLaunchKernelGGL(debug_decode_kernel, dim3((E + 255) / 256, batch->num_reqs), dim3(256), 0, stream,
                     batch->block_tables, batch->num_entries, batch->ctx_lens, E, out);
  return launched();
}

}  // extern "C"
