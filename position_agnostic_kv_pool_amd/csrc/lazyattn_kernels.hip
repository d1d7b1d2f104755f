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
//  - decode: each key row r of a block starting at S is rotated by
//    R(S - p + r) = R(S - p) R(r); R(S - p) is formed once per block and
//    R(r) is a per-lane constant (gist.science, Technical Implementation >
//    Decoding: the rotation is fused into the inner loop; only K and V are
//    read, the block metadata is one 64-bit word).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

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

// Rotate the interleaved channel pair held in one 32-bit bf16x2 word.
__device__ __forceinline__ uint32_t rotate_pair(uint32_t u, float2 ph) {
  const float x0 = bf_lo(u), x1 = bf_hi(u);
  return pack_bf16x2(x0 * ph.x - x1 * ph.y, x0 * ph.y + x1 * ph.x);
}

struct EntryInfo {
  uint32_t blk;
  int32_t start;
  int32_t len;
};

// Decode table entry e of a request: block id, logical start and valid length
// (next entry's start, or the context length for the last entry).
__device__ __forceinline__ EntryInfo entry_info(const uint64_t* row, int e, int n_ent, int ctx) {
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

// Split-K completion: every work-group of a tile publishes its partial
// result, then increments the tile's counter; the one that brings it to
// `splits` sees every partial and merges them.  Device-scope fences order the
// partial stores before the increment and the merge loads after it (the
// XCDs' L2 caches are not coherent with each other without them).
__device__ __forceinline__ bool arrive_last(unsigned* counter, int splits) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(counter, 1u) == static_cast<unsigned>(splits - 1);
  __syncthreads();
  if (!s_last) return false;
  __threadfence();
  return true;
}

// ---------------------------------------------------------------------------
// Prefill, bf16, MFMA.
//
// Work-group = 8 waves = 256 query rows: the G heads of one KV group at
// m_q = 256 / G consecutive positions (row rho -> position rho / G, head
// rho % G).  Each wave owns 32 rows as two 16-row tiles.  A key tile is four
// table entries (64 key slots).  Per tile:
//   S^T (keys x rows) = K~ (keys x D) . Q~^T          16x16x32 MFMA, K~ from LDS
//   online softmax over the keys of each row (base 2, scale folded into Q~)
//   O^T (D x rows)   += V^T (D x keys) . P^T         16x16x32 MFMA, V^T from LDS
// The S^T accumulator leaves each lane with 4 consecutive keys of one row,
// which is exactly a P^T operand slice, so P never leaves registers.
// ---------------------------------------------------------------------------
struct PrefillArgs {
  const uint16_t* q;
  const int32_t* cu_q;
  const uint16_t* kpool;
  const uint16_t* vpool;
  const uint64_t* tables;
  const int32_t* n_ent;
  const int32_t* ctx;
  const float* alibi;
  uint16_t* out;
  float* o_part;
  float* ml_part;
  unsigned* counters;
  int32_t Hq, Hkv, G, max_entries, total_q, m_q, eps, splits;
  float scale_log2;
  RopeRev rope;
};

constexpr int kPD = 128;        // head dim of the bf16 kernels
constexpr int kKS = kPD + 8;    // K tile row stride in bf16 (272 B: conflict-free 16-lane reads)
constexpr int kVS = 40;         // V tile row stride in bf16 (80 B)

template <int PE>
__global__ __launch_bounds__(512) void prefill_bf16_kernel(const PrefillArgs A) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * kKS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * kPD * kVS];
  __shared__ __attribute__((aligned(16))) float2 base_s[2][4][64];
  __shared__ __attribute__((aligned(16))) float2 rtab[16][64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int qt = blockIdx.x, r = blockIdx.y;
  const int kvh = blockIdx.z % A.Hkv, split = blockIdx.z / A.Hkv;
  const int q0 = A.cu_q[r];
  const int q_len = A.cu_q[r + 1] - q0;
  const int m0 = qt * A.m_q;
  if (m0 >= q_len) return;
  const int L = A.ctx[r];
  const int ne = A.n_ent[r];
  const int p0 = L - q_len + m0;                      // position of the tile's first row
  const int mq = min(A.m_q, q_len - m0);
  const int p_last = p0 + mq - 1;
  const uint64_t* trow = A.tables + static_cast<size_t>(r) * A.max_entries;
  const int e_begin = split * A.eps;
  const int e_end = min(ne, e_begin + A.eps);
  const int G = A.G, Hq = A.Hq, Hkv = A.Hkv;

  // ---- rows owned by this lane, and the query fragments -------------------
  int p_row[2], tok[2], head[2];
  bool row_ok[2];
  float slope[2];
  bf16x8 qf[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int rho = wave * 32 + nt * 16 + n;
    const int m = rho / G, gh = rho - m * G;
    row_ok[nt] = m < mq;
    p_row[nt] = p0 + m;
    tok[nt] = q0 + m0 + m;
    head[nt] = kvh * G + gh;
    slope[nt] = (PE == LAZYATTN_PE_ALIBI) ? alibi_slope(A.alibi, head[nt], Hq) * kLog2e : 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (row_ok[nt])
        raw = *reinterpret_cast<const uint4*>(A.q + (static_cast<size_t>(tok[nt]) * Hq + head[nt]) * kPD +
                                              32 * s + 8 * g);
      uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float x0 = bf_lo(w4[jj]), x1 = bf_hi(w4[jj]);
        if (PE == LAZYATTN_PE_ROPE) {
          const float2 ph = unit_phase(m, A.rope.rev[16 * s + 4 * g + jj]);
          const float y0 = x0 * ph.x - x1 * ph.y;
          const float y1 = x0 * ph.y + x1 * ph.x;
          x0 = y0;
          x1 = y1;
        }
        w4[jj] = pack_bf16x2(x0 * A.scale_log2, x1 * A.scale_log2);
      }
      qf[nt][s] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
    }
  }

  // ---- per-lane key rotation table R(r) for r = 0..15 ----------------------
  if (PE == LAZYATTN_PE_ROPE) {
    for (int i = tid; i < 16 * 64; i += 512) rtab[i >> 6][i & 63] = unit_phase(i >> 6, A.rope.rev[i & 63]);
  }

  // staging roles: thread -> (entry se, key row sr, channel chunk sc) for K,
  //                thread -> (entry se, channel sd) for V
  const int se = tid >> 7, sr = (tid >> 3) & 15, sc = tid & 7, sd = tid & 127;

  f32x4 O[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt][0] = O[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};

  // entries of tile starting at et: valid when inside the split, in the table
  // and not entirely after the tile's last query position
  auto tile_entry = [&](int et, int i, EntryInfo& inf) -> bool {
    const int e = et + i;
    if (e >= e_end) return false;
    inf = entry_info(trow, e, ne, L);
    return inf.start <= p_last;
  };

  uint4 kr0 = make_uint4(0, 0, 0, 0), kr1 = kr0, vr0 = kr0, vr1 = kr0;
  auto load_tile = [&](int et) {
    EntryInfo inf;
    if (tile_entry(et, se, inf)) {
      const uint16_t* kb = A.kpool + (static_cast<size_t>(inf.blk) * Hkv + kvh) * (kBlock * kPD);
      const uint4* kp = reinterpret_cast<const uint4*>(kb + sr * kPD + 16 * sc);
      kr0 = kp[0];
      kr1 = kp[1];
      const uint16_t* vb = A.vpool + (static_cast<size_t>(inf.blk) * Hkv + kvh) * (kPD * kBlock);
      const uint4* vp = reinterpret_cast<const uint4*>(vb + sd * kBlock);
      vr0 = vp[0];
      vr1 = vp[1];
    }
  };
  auto tile_bases = [&](int et, int buf) {
    if (PE == LAZYATTN_PE_ROPE && tid < 256) {
      const int e = tid >> 6, pr = tid & 63;
      EntryInfo inf;
      float2 ph = make_float2(1.f, 0.f);
      if (tile_entry(et, e, inf)) ph = unit_phase(inf.start - p0, A.rope.rev[pr]);
      base_s[buf][e][pr] = ph;
    }
  };

  int et = e_begin;
  bool have = e_begin < e_end && entry_info(trow, e_begin, ne, L).start <= p_last;
  if (have) {
    load_tile(et);
    tile_bases(et, 0);
  }
  __syncthreads();

  for (int it = 0; have; ++it) {
    const int buf = it & 1;
    // ---- stage tile `et` into LDS: rotate K, transpose V into MFMA order --
    {
      EntryInfo inf;
      const bool ok = tile_entry(et, se, inf);
      const int len = ok ? inf.len : 0;
      // K: rows past the entry's length are written as zeros
      uint32_t kw[8] = {kr0.x, kr0.y, kr0.z, kr0.w, kr1.x, kr1.y, kr1.z, kr1.w};
      if (sr >= len) {
#pragma unroll
        for (int i = 0; i < 8; ++i) kw[i] = 0;
      } else if (PE == LAZYATTN_PE_ROPE) {
#pragma unroll
        for (int i = 0; i < 8; ++i) kw[i] = rotate_pair(kw[i], cmul(base_s[buf][se][8 * sc + i], rtab[sr][8 * sc + i]));
      }
      uint4* kd = reinterpret_cast<uint4*>(&Ks[(16 * se + sr) * kKS + 16 * sc]);
      kd[0] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
      kd[1] = make_uint4(kw[4], kw[5], kw[6], kw[7]);
      // V: channel sd of entry se, keys 4gg..4gg+3 -> Vs[se/2][sd][gg*8 + (se&1)*4 ..]
      uint32_t vw[8] = {vr0.x, vr0.y, vr0.z, vr0.w, vr1.x, vr1.y, vr1.z, vr1.w};
      if (len < kBlock) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k0 = 2 * i, k1 = 2 * i + 1;
          uint32_t lo = (k0 < len) ? (vw[i] & 0xffffu) : 0u;
          uint32_t hi = (k1 < len) ? (vw[i] & 0xffff0000u) : 0u;
          vw[i] = lo | hi;
        }
      }
      uint16_t* vrow = &Vs[((se >> 1) * kPD + sd) * kVS + (se & 1) * 4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        *reinterpret_cast<uint2*>(vrow + gg * 8) = make_uint2(vw[2 * gg], vw[2 * gg + 1]);
    }
    // ---- prefetch the next tile ---------------------------------------------
    const int et_next = et + 4;
    const bool have_next = et_next < e_end && entry_info(trow, et_next, ne, L).start <= p_last;
    if (have_next) {
      load_tile(et_next);
      tile_bases(et_next, buf ^ 1);
    }
    __syncthreads();

    // ---- tile masks (wave-uniform) --------------------------------------------
    int t_start[4], t_len[4];
    bool full = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      EntryInfo inf;
      if (tile_entry(et, i, inf)) {
        t_start[i] = inf.start;
        t_len[i] = inf.len;
      } else {
        t_start[i] = 0;
        t_len[i] = 0;
      }
      full = full && t_len[i] == kBlock;
    }
    full = full && (t_start[3] + kBlock - 1 <= p0);

    // ---- S^T = K~ Q~^T ---------------------------------------------------------
    f32x4 S[4][2];
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      S[tau][0] = S[tau][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(16 * tau + n) * kKS + 32 * s + 8 * g]);
        S[tau][0] = mfma16x16x32(a, qf[0][s], S[tau][0]);
        S[tau][1] = mfma16x16x32(a, qf[1][s], S[tau][1]);
      }
    }

    // ---- online softmax, per row ------------------------------------------------
    uint32_t pk[4][2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = kNegInf;
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v = S[tau][nt][j];
          const int kr = 4 * g + j;
          const int t = t_start[tau] + kr;
          if (!full) {
            const bool vis = (kr < t_len[tau]) && (t <= p_row[nt]);
            v = vis ? v : kNegInf;
          }
          if (PE == LAZYATTN_PE_ALIBI) v -= slope[nt] * static_cast<float>(p_row[nt] - t);
          S[tau][nt][j] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
      // the row sum uses the bf16-rounded weights that enter P.V, so the
      // output is an exact convex combination of the V rows
      float rs = 0.f;
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        float pe[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) pe[j] = __builtin_amdgcn_exp2f(S[tau][nt][j] - m_use);
        pk[tau][nt][0] = pack_bf16x2(pe[0], pe[1]);
        pk[tau][nt][1] = pack_bf16x2(pe[2], pe[3]);
        rs += (bf_lo(pk[tau][nt][0]) + bf_hi(pk[tau][nt][0])) + (bf_lo(pk[tau][nt][1]) + bf_hi(pk[tau][nt][1]));
      }
      l_run[nt] = l_run[nt] * alpha + rs;
      m_run[nt] = m_new;
      if (alpha != 1.0f) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) O[dt][nt] *= alpha;
      }
    }

    // ---- O^T += V^T P^T -----------------------------------------------------------
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 b0 = __builtin_bit_cast(bf16x8, make_uint4(pk[2 * u][0][0], pk[2 * u][0][1], pk[2 * u + 1][0][0], pk[2 * u + 1][0][1]));
      bf16x8 b1 = __builtin_bit_cast(bf16x8, make_uint4(pk[2 * u][1][0], pk[2 * u][1][1], pk[2 * u + 1][1][0], pk[2 * u + 1][1][1]));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Vs[(u * kPD + 16 * dt + n) * kVS + 8 * g]);
        O[dt][0] = mfma16x16x32(a, b0, O[dt][0]);
        O[dt][1] = mfma16x16x32(a, b1, O[dt][1]);
      }
    }
    __syncthreads();
    et = et_next;
    have = have_next;
  }

  // ---- epilogue ------------------------------------------------------------------
  float lt[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    lt[nt] = l_run[nt] + __shfl_xor(l_run[nt], 16);
    lt[nt] += __shfl_xor(lt[nt], 32);
  }
  if (A.splits == 1) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (!row_ok[nt]) continue;
      const size_t rowoff = static_cast<size_t>(tok[nt]) * Hq + head[nt];
      const float inv = 1.0f / lt[nt];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 o = O[dt][nt];
        *reinterpret_cast<uint2*>(A.out + rowoff * kPD + 16 * dt + 4 * g) =
            make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
      }
    }
    return;
  }
  // Split keys: publish this split's (o, m, l); the last work-group of the
  // tile to arrive merges all splits with log-sum-exp weights.
  const size_t rows_total = static_cast<size_t>(A.total_q) * Hq;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (!row_ok[nt]) continue;
    const size_t prow = static_cast<size_t>(split) * rows_total + static_cast<size_t>(tok[nt]) * Hq + head[nt];
    if (lt[nt] > 0.f) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4*>(A.o_part + prow * kPD + 16 * dt + 4 * g) = O[dt][nt];
    }
    if (g == 0) *reinterpret_cast<float2*>(A.ml_part + prow * 2) = make_float2(m_run[nt], lt[nt]);
  }
  const unsigned tile = (static_cast<unsigned>(qt) * gridDim.y + r) * Hkv + kvh;
  if (!arrive_last(A.counters + tile, A.splits)) return;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (!row_ok[nt]) continue;
    const size_t rowoff = static_cast<size_t>(tok[nt]) * Hq + head[nt];
    // merge in split order whichever work-group arrived last, so the result
    // is bit-for-bit reproducible; this work-group's own partial comes from
    // registers, which hold exactly what it stored
    float M = kNegInf;
    for (int sp = 0; sp < A.splits; ++sp)
      M = fmaxf(M, sp == split ? m_run[nt] : A.ml_part[(static_cast<size_t>(sp) * rows_total + rowoff) * 2]);
    float Lsum = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < A.splits; ++sp) {
      const size_t prow = static_cast<size_t>(sp) * rows_total + rowoff;
      const float2 ml = sp == split ? make_float2(m_run[nt], lt[nt])
                                    : *reinterpret_cast<const float2*>(A.ml_part + prow * 2);
      if (ml.x == kNegInf) continue;
      const float w = __builtin_amdgcn_exp2f(ml.x - M);
      Lsum = fmaf(w, ml.y, Lsum);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 o = sp == split ? O[dt][nt] : *reinterpret_cast<const f32x4*>(A.o_part + prow * kPD + 16 * dt + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[dt][j] = fmaf(w, o[j], acc[dt][j]);
      }
    }
    const float inv = 1.0f / Lsum;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<uint2*>(A.out + rowoff * kPD + 16 * dt + 4 * g) =
          make_uint2(pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv), pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv));
  }
  if (tid == 0) A.counters[tile] = 0u;  // leave the counter ready for the next call
}

// ---------------------------------------------------------------------------
// Decode, bf16, MFMA, split-K over table entries.
//
// Work-group = 4 waves for one (request, KV head, split); wave w takes
// entries e_begin + w, + 4, ...  Per block (16 keys) a wave computes
//   S^T (16 keys x 16 heads) = K~ (16 x D) . q^T            4 x 16x16x32 MFMA
//   O^T (D x 16 heads)      += V^T (D x 16 keys) . P^T      8 x 16x16x16 MFMA
// with the group's G heads padded to NT tiles of 16.  Lane (g, n) loads key
// row n, channels 32g..32g+31 (64 contiguous bytes) and V channel rows
// 16dt + n, keys 4g..4g+3 (8 bytes each); the whole 8 KB block is read once.
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kpool;
  const uint16_t* vpool;
  const uint64_t* tables;
  const int32_t* n_ent;
  const int32_t* ctx;
  const float* alibi;
  uint16_t* out;
  float* o_part;
  float* ml_part;
  unsigned* counters;
  int32_t R, Hq, Hkv, G, max_entries, eps, splits;
  float scale_log2;
  RopeRev rope;
};

constexpr int kOS = kPD + 4;  // LDS row stride (floats) of the wave-merge buffer

template <int PE, int NT>
__global__ __launch_bounds__(256) void decode_bf16_kernel(const DecodeArgs A) {
  extern __shared__ __attribute__((aligned(16))) float dsm[];
  float2* bsh = reinterpret_cast<float2*>(dsm);             // [4 waves][2][64]
  float* ml_s = dsm + 4 * 2 * 64 * 2;                         // [4][NT*16][2]
  float* o_s = ml_s + 4 * NT * 16 * 2;                        // [4][G][kOS]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int split = blockIdx.x, kvh = blockIdx.y, r = blockIdx.z;
  const int G = A.G, Hq = A.Hq, Hkv = A.Hkv;
  const int L = A.ctx[r];
  const int p = L - 1;
  const int ne = A.n_ent[r];
  const uint64_t* trow = A.tables + static_cast<size_t>(r) * A.max_entries;
  const int e_begin = split * A.eps;
  const int e_end = min(ne, e_begin + A.eps);

  // query fragments: lane (g, n) holds head column nt*16+n, channels 32g + 8s + 0..7
  bf16x8 qb[NT][4];
  float slope[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + n;
    const bool ok = col < G;
    const int h = kvh * G + (ok ? col : 0);
    slope[nt] = (PE == LAZYATTN_PE_ALIBI) ? alibi_slope(A.alibi, h, Hq) * kLog2e : 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (ok) raw = *reinterpret_cast<const uint4*>(A.q + (static_cast<size_t>(r) * Hq + h) * kPD + 32 * g + 8 * s);
      qb[nt][s] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  // R(n) for this lane's key row and pairs 16g..16g+15; this lane's pair for R(S - p)
  float2 rt[16];
  double my_rev = 0.0;
  if (PE == LAZYATTN_PE_ROPE) {
#pragma unroll
    for (int i = 0; i < 16; ++i) rt[i] = unit_phase(n, A.rope.rev[16 * g + i]);
    my_rev = A.rope.rev[lane];
  }

  f32x4 O[8][NT];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = kNegInf;
    l_run[nt] = 0.f;
  }

  uint4 kr[4];
  uint2 vr[8];
  EntryInfo cur;
  auto load_block = [&](int e, EntryInfo& inf, uint4 (&k)[4], uint2 (&v)[8]) {
    inf = entry_info(trow, e, ne, L);
    const uint16_t* kb = A.kpool + (static_cast<size_t>(inf.blk) * Hkv + kvh) * (kBlock * kPD);
    const uint4* kp = reinterpret_cast<const uint4*>(kb + n * kPD + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) k[s] = kp[s];
    const uint16_t* vb = A.vpool + (static_cast<size_t>(inf.blk) * Hkv + kvh) * (kPD * kBlock);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) v[dt] = *reinterpret_cast<const uint2*>(vb + (16 * dt + n) * kBlock + 4 * g);
  };

  int e = e_begin + wave;
  if (e < e_end) load_block(e, cur, kr, vr);
  for (int it = 0; e < e_end; ++it) {
    const EntryInfo inf = cur;
    uint4 k[4] = {kr[0], kr[1], kr[2], kr[3]};
    uint2 v[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) v[dt] = vr[dt];
    const int e_next = e + 4;
    if (e_next < e_end) load_block(e_next, cur, kr, vr);

    // ---- rotate the key rows: R(S - p + n) = R(S - p) R(n) ------------------
    bf16x8 ka[4];
    if (PE == LAZYATTN_PE_ROPE) {
      float2* bw = bsh + (wave * 2 + (it & 1)) * 64;
      bw[lane] = unit_phase(inf.start - p, my_rev);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t w4[4] = {k[s].x, k[s].y, k[s].z, k[s].w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int i = 4 * s + jj;                      // pair 16g + i
          w4[jj] = rotate_pair(w4[jj], cmul(bw[16 * g + i], rt[i]));
        }
        ka[s] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = __builtin_bit_cast(bf16x8, k[s]);
    }
    if (n >= inf.len) {
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
    if (inf.len < kBlock) {
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
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) S = mfma16x16x32(ka[s], qb[nt][s], S);
      float mx = kNegInf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int krow = 4 * g + j;
        float x = (krow < inf.len) ? S[j] * A.scale_log2 : kNegInf;
        if (PE == LAZYATTN_PE_ALIBI) x -= slope[nt] * static_cast<float>(p - (inf.start + krow));
        S[j] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
      float pe[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pe[j] = __builtin_amdgcn_exp2f(S[j] - m_use);
      const uint32_t p01 = pack_bf16x2(pe[0], pe[1]), p23 = pack_bf16x2(pe[2], pe[3]);
      // row sum of the bf16-rounded weights that enter P.V
      const float rs = (bf_lo(p01) + bf_hi(p01)) + (bf_lo(p23) + bf_hi(p23));
      l_run[nt] = l_run[nt] * alpha + rs;
      m_run[nt] = m_new;
      const s16x4 pb = __builtin_bit_cast(s16x4, make_uint2(p01, p23));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        O[dt][nt] = mfma16x16x16(__builtin_bit_cast(s16x4, v[dt]), pb, O[dt][nt] * alpha);
      }
    }
    e = e_next;
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
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + n;
    if (col >= G) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_s[(w * NT * 16 + col) * 2]);
    const float f = (M == kNegInf || m_run[nt] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run[nt] - M);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<f32x4*>(o_s + (wave * G + col) * kOS + 16 * dt + 4 * g) = O[dt][nt] * f;
  }
  __syncthreads();
  for (int idx = tid; idx < G * kPD; idx += 256) {
    const int col = idx / kPD, d = idx - col * kPD;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_s[(w * NT * 16 + col) * 2]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = ml_s[(w * NT * 16 + col) * 2];
      if (M != kNegInf && mw != kNegInf) lsum += __builtin_amdgcn_exp2f(mw - M) * ml_s[(w * NT * 16 + col) * 2 + 1];
      osum += o_s[(w * G + col) * kOS + d];
    }
    const int h = kvh * G + col;
    const size_t rowoff = static_cast<size_t>(r) * Hq + h;
    if (A.splits == 1) {
      const float val = lsum > 0.f ? osum / lsum : 0.f;
      A.out[rowoff * kPD + d] = static_cast<uint16_t>(pack_bf16x2(val, 0.f) & 0xffffu);
    } else {
      const size_t prow = static_cast<size_t>(split) * A.R * Hq + rowoff;
      A.o_part[prow * kPD + d] = osum;
      if (d == 0) *reinterpret_cast<float2*>(A.ml_part + prow * 2) = make_float2(M, lsum);
    }
  }
  if (A.splits == 1) return;
  // the last split of this (request, KV head) to finish merges all splits
  const unsigned tile = static_cast<unsigned>(r) * Hkv + kvh;
  if (!arrive_last(A.counters + tile, A.splits)) return;
  const size_t rows_total = static_cast<size_t>(A.R) * Hq;
  for (int idx = tid; idx < G * kPD; idx += 256) {
    const int col = idx / kPD, d = idx - col * kPD;
    const size_t rowoff = static_cast<size_t>(r) * Hq + kvh * G + col;
    float M = kNegInf;
    for (int sp = 0; sp < A.splits; ++sp) M = fmaxf(M, A.ml_part[(sp * rows_total + rowoff) * 2]);
    float lsum = 0.f, osum = 0.f;
    if (M != kNegInf) {
      for (int sp = 0; sp < A.splits; ++sp) {
        const size_t prow = sp * rows_total + rowoff;
        const float2 ml = *reinterpret_cast<const float2*>(A.ml_part + prow * 2);
        if (ml.x == kNegInf) continue;
        const float w = __builtin_amdgcn_exp2f(ml.x - M);
        lsum = fmaf(w, ml.y, lsum);
        osum = fmaf(w, A.o_part[prow * kPD + d], osum);
      }
    }
    const float val = lsum > 0.f ? osum / lsum : 0.f;
    A.out[rowoff * kPD + d] = static_cast<uint16_t>(pack_bf16x2(val, 0.f) & 0xffffu);
  }
  if (tid == 0) A.counters[tile] = 0u;  // leave the counter ready for the next call
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

static size_t decode_lds_bytes(int nt, int group) {
  return (4 * 2 * 64 * 2 + 4 * nt * 16 * 2 + 4 * static_cast<size_t>(group) * kOS) * sizeof(float);
}

}  // namespace lazyattn

using namespace lazyattn;

extern "C" {

lazyattn_status lazyattn_prefill(const lazyattn_config* cfg, const void* q, const int32_t* cu_q_lens,
                                 int32_t total_q, int32_t max_q_len, const void* k_pool, const void* v_pool,
                                 int64_t num_blocks, const lazyattn_batch* batch, int32_t num_splits, void* out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if ((st = check_batch(batch)) != LAZYATTN_OK) return st;
  if (total_q < 0 || max_q_len < 0 || num_splits < 0 || num_splits > 64 || num_blocks < 0) return LAZYATTN_EINVAL;
  if (batch->num_reqs == 0 || total_q == 0) return LAZYATTN_OK;
  if (!q || !cu_q_lens || !k_pool || !v_pool || !out || num_blocks < 1 || max_q_len < 1) return LAZYATTN_EINVAL;
  const int R = batch->num_reqs, Hq = cfg->num_q_heads, Hkv = cfg->num_kv_heads, G = Hq / Hkv;
  const RopeRev rope = make_rope_rev(cfg);
  const float scale = softmax_scale_of(cfg);

  if (cfg->dtype == LAZYATTN_F32) {
    if (max_q_len > 65535 * 64) return LAZYATTN_EUNSUPPORTED;
    NaiveArgs a{static_cast<const float*>(q), cu_q_lens, static_cast<const float*>(k_pool),
                static_cast<const float*>(v_pool), batch->block_tables, batch->num_entries, batch->ctx_lens,
                cfg->alibi_slopes, static_cast<float*>(out), Hq, Hkv, G, cfg->head_dim, batch->max_entries,
                cfg->pe, scale, rope};
    if (R > 65535 || Hq > 65535) return LAZYATTN_EUNSUPPORTED;
    hipLaunchKernelGGL(attn_f32_kernel, dim3(max_q_len, R, Hq), dim3(64), 0, stream, a);
    return launched();
  }

  if (G > 256) return LAZYATTN_EUNSUPPORTED;
  const int splits = num_splits > 0 ? num_splits : choose_prefill_splits(cfg, R, max_q_len, batch->max_entries);
  const size_t need = lazyattn_prefill_workspace_size(cfg, R, total_q, max_q_len, batch->max_entries, splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return LAZYATTN_EWORKSPACE;
  const int m_q = prefill_positions_per_tile(G);
  const long long gx = (max_q_len + m_q - 1) / m_q;
  const long long gz = static_cast<long long>(Hkv) * splits;
  if (R > 65535 || gz > 65535 || gx > 0x7fffffff) return LAZYATTN_EUNSUPPORTED;
  if (splits > 1 && gx * R * Hkv > kMaxSplitTiles) return LAZYATTN_EUNSUPPORTED;
  unsigned* counters = splits > 1 ? static_cast<unsigned*>(workspace) : nullptr;
  float* o_part = splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes) : nullptr;
  float* ml_part = splits > 1 ? o_part + static_cast<size_t>(splits) * total_q * Hq * kPD : nullptr;
  PrefillArgs a{static_cast<const uint16_t*>(q), cu_q_lens, static_cast<const uint16_t*>(k_pool),
                static_cast<const uint16_t*>(v_pool), batch->block_tables, batch->num_entries, batch->ctx_lens,
                cfg->alibi_slopes, static_cast<uint16_t*>(out), o_part, ml_part, counters, Hq, Hkv, G,
                batch->max_entries,
                total_q, m_q, prefill_entries_per_split(batch->max_entries, splits), splits, scale * kLog2e, rope};
  const dim3 grid(static_cast<unsigned>(gx), R, static_cast<unsigned>(gz));
  switch (cfg->pe) {
    case LAZYATTN_PE_ROPE: hipLaunchKernelGGL(prefill_bf16_kernel<LAZYATTN_PE_ROPE>, grid, dim3(512), 0, stream, a); break;
    case LAZYATTN_PE_NONE: hipLaunchKernelGGL(prefill_bf16_kernel<LAZYATTN_PE_NONE>, grid, dim3(512), 0, stream, a); break;
    default: hipLaunchKernelGGL(prefill_bf16_kernel<LAZYATTN_PE_ALIBI>, grid, dim3(512), 0, stream, a); break;
  }
  return launched();
}

lazyattn_status lazyattn_decode(const lazyattn_config* cfg, const void* q, const void* k_pool, const void* v_pool,
                                int64_t num_blocks, const lazyattn_batch* batch, int32_t num_splits, void* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  lazyattn_status st = check_config(cfg);
  if (st != LAZYATTN_OK) return st;
  if ((st = check_batch(batch)) != LAZYATTN_OK) return st;
  if (num_splits < 0 || num_splits > 256 || num_blocks < 0) return LAZYATTN_EINVAL;
  if (batch->num_reqs == 0) return LAZYATTN_OK;
  if (!q || !k_pool || !v_pool || !out || num_blocks < 1) return LAZYATTN_EINVAL;
  const int R = batch->num_reqs, Hq = cfg->num_q_heads, Hkv = cfg->num_kv_heads, G = Hq / Hkv;
  const RopeRev rope = make_rope_rev(cfg);
  const float scale = softmax_scale_of(cfg);

  if (cfg->dtype == LAZYATTN_F32) {
    NaiveArgs a{static_cast<const float*>(q), nullptr, static_cast<const float*>(k_pool),
                static_cast<const float*>(v_pool), batch->block_tables, batch->num_entries, batch->ctx_lens,
                cfg->alibi_slopes, static_cast<float*>(out), Hq, Hkv, G, cfg->head_dim, batch->max_entries,
                cfg->pe, scale, rope};
    if (R > 65535 || Hq > 65535) return LAZYATTN_EUNSUPPORTED;
    hipLaunchKernelGGL(attn_f32_kernel, dim3(1, R, Hq), dim3(64), 0, stream, a);
    return launched();
  }

  if (G > 32) return LAZYATTN_EUNSUPPORTED;
  const int splits = num_splits > 0 ? num_splits : choose_decode_splits(cfg, R, batch->max_entries);
  const size_t need = lazyattn_decode_workspace_size(cfg, R, batch->max_entries, splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return LAZYATTN_EWORKSPACE;
  if (R > 65535 || Hkv > 65535) return LAZYATTN_EUNSUPPORTED;
  if (splits > 1 && static_cast<long long>(R) * Hkv > kMaxSplitTiles) return LAZYATTN_EUNSUPPORTED;
  unsigned* counters = splits > 1 ? static_cast<unsigned*>(workspace) : nullptr;
  float* o_part = splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes) : nullptr;
  float* ml_part = splits > 1 ? o_part + static_cast<size_t>(splits) * R * Hq * kPD : nullptr;
  DecodeArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_pool),
               static_cast<const uint16_t*>(v_pool), batch->block_tables, batch->num_entries, batch->ctx_lens,
               cfg->alibi_slopes, static_cast<uint16_t*>(out), o_part, ml_part, counters, R, Hq, Hkv, G,
               batch->max_entries, decode_entries_per_split(batch->max_entries, splits), splits, scale * kLog2e,
               rope};
  const dim3 grid(splits, Hkv, R);
  const int nt = G <= 16 ? 1 : 2;
  const size_t lds = decode_lds_bytes(nt, G);
#define LAZYATTN_DECODE(PEV, NTV)                                                                     \
  do {                                                                                              \
    if (lds > 65536)                                                                                \
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_bf16_kernel<PEV, NTV>),       \
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)); \
    hipLaunchKernelGGL((decode_bf16_kernel<PEV, NTV>), grid, dim3(256), lds, stream, a);            \
  } while (0)
  if (nt == 1) {
    switch (cfg->pe) {
      case LAZYATTN_PE_ROPE: LAZYATTN_DECODE(LAZYATTN_PE_ROPE, 1); break;
      case LAZYATTN_PE_NONE: LAZYATTN_DECODE(LAZYATTN_PE_NONE, 1); break;
      default: LAZYATTN_DECODE(LAZYATTN_PE_ALIBI, 1); break;
    }
  } else {
    switch (cfg->pe) {
      case LAZYATTN_PE_ROPE: LAZYATTN_DECODE(LAZYATTN_PE_ROPE, 2); break;
      case LAZYATTN_PE_NONE: LAZYATTN_DECODE(LAZYATTN_PE_NONE, 2); break;
      default: LAZYATTN_DECODE(LAZYATTN_PE_ALIBI, 2); break;
    }
  }
#undef LAZYATTN_DECODE
  return launched();
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
  if (cfg->dtype == LAZYATTN_BF16) {
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
