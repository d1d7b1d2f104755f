/*
 * lazyattn.h - attention over a position-agnostic paged KV pool with RoPE
 * applied lazily inside the kernels (MI355X / gfx950).
 *
 * The method is LazyAttention ("LazyAttention: Efficient Retrieval-Augmented
 * Generation with Deferred Positional Encoding", arXiv 2606.04302).  Its pages
 * say: the KV cache stores content-only keys and values and positional
 * information is applied on the fly inside the attention kernel (gist.science
 * explainer, Technical Summary > Methodology > Core Concept); one physical KV
 * copy then serves many logical requests at arbitrary positions (shd-paper.top
 * digest, original English abstract); the result equals attention over keys
 * re-encoded at their positions, because RoPE scores depend only on the
 * relative offset (gist.science, Mathematical Equivalence); per-block metadata
 * (block id, offset) is bit-packed into one register-sized word (gist.science,
 * Technical Implementation > Decoding).
 *
 * Conventions for every entry point below:
 *  - Ownership: the caller owns every buffer.  The library never allocates or
 *    frees device memory and keeps no per-call state.
 *  - Asynchrony: GPU calls enqueue work on `stream` and return; the library
 *    never synchronises.  Buffers must stay alive until the stream passes.
 *  - Pointers: "device" pointers address GPU memory of the current device;
 *    "host" pointers address CPU memory and are read before the call returns.
 *  - Access: the K/V pools are read-only to prefill and decode (shared blocks
 *    are never written); `out` must not alias any input.
 *  - Errors: argument errors detectable on the host return LAZYATTN_EINVAL or
 *    LAZYATTN_EUNSUPPORTED before any launch; a short workspace returns
 *    LAZYATTN_EWORKSPACE; a failed launch returns LAZYATTN_EHIP.  Device-side
 *    contract violations (a malformed table) are undefined behaviour; check
 *    host copies with lazyattn_validate_tables.  No C++ exception crosses
 *    this interface.
 *
 * Data layout (B = block_size = 16, D = head_dim, Hkv = KV heads, Hq = query
 * heads, G = Hq / Hkv; element type = config dtype for the plain pool format):
 *  - K pool  [num_blocks][Hkv][B][D]   one block = B token rows of D channels
 *  - V pool  [num_blocks][Hkv][D][B]   one block = D channel rows of B tokens
 *    By default both hold content only: keys are never rotated in storage.
 *    Two variants are selected per call: keys in document-local frames
 *    (lazyattn_batch.frame_starts, "Key frames" below) and an FP8 chunk
 *    format (lazyattn_config.kv_format, "Pool formats" below).
 *  - Table word (uint64): bits 63..32 logical start, bits 31..0 block id.
 *    A request's words are ordered by logical start; the context is dense:
 *    entry e covers logical positions [start_e, start_{e+1}) (the last one
 *    up to ctx_len), 1 <= length <= B, first start 0.  Rows of a block past
 *    the entry's length are padding and are never read into a result.
 *  - Query head h reads KV head h / G.
 *  - RoPE pairs are interleaved channels (2i, 2i+1), frequency
 *    theta^(-2i/D) or the caller's table (lazyattn_config.rope_inv_freq); a
 *    query at position p and a key at t score scale * q^T R(t - p) k.
 */
#ifndef LAZYATTN_H
#define LAZYATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LAZYATTN_ABI_VERSION 9

typedef enum {
  LAZYATTN_OK = 0,
  LAZYATTN_EINVAL = 1,        /* bad argument (null pointer, inconsistent sizes) */
  LAZYATTN_EUNSUPPORTED = 2,  /* valid but not built (head_dim, block_size, dtype, group size) */
  LAZYATTN_EWORKSPACE = 3,    /* workspace smaller than the matching *_workspace_size */
  LAZYATTN_EHIP = 4           /* a HIP launch failed */
} lazyattn_status;

typedef enum { LAZYATTN_F32 = 0, LAZYATTN_BF16 = 1 } lazyattn_dtype;

/* Positional encoding applied inside the kernels.  NONE is the rotation-free
 * control; ALIBI adds -slope_h * (p - t) to the scaled score (gist.science,
 * Key Contributions > Generalizability, names ALiBi among compatible
 * encodings). */
typedef enum { LAZYATTN_PE_ROPE = 0, LAZYATTN_PE_NONE = 1, LAZYATTN_PE_ALIBI = 2 } lazyattn_pe;

/* Config flags.  EXACT_MAX: the bf16 prefill first computes every query
 * row's exact score maximum over its keys (a scores-only pass) and uses it as
 * the softmax reference, instead of taking the reference from the first key
 * tile and redoing only when a later score outgrows it; same results up to
 * rounding, for validation. */
#define LAZYATTN_FLAG_EXACT_MAX 1

/* Where the bf16 prefill turns the keys of a content-only pool (pe ROPE, plain
 * pool, no frame_starts).  The pages rotate each staged key tile inside the
 * attention kernel (gist.science, Technical Implementation > Prefilling), so a
 * chunk of many query tiles turns the same key once per query tile.  With
 * KEYS_ONCE the call first turns every key of every request once, by
 * R(t - c_r) with c_r = ctx_lens[r] - q_len_r (the position of the request's
 * first new token), into the workspace, then attends with the queries turned
 * by R(m - c_r) and no rotation in the attention kernel; the pool itself is
 * never written.  KEYS_FUSED keeps the rotation inside the attention kernel.
 * With neither flag the library turns the keys once when a request spans at
 * least LAZYATTN_KEYS_ONCE_TILES query tiles of 256 rows (ceil(max_q_len /
 * floor(256 / G)) >= 8), where it measured faster.  The choice is made per
 * call from max_q_len, so in a batch mixing one long chunk with short requests
 * every request's keys are turned once (the short ones gain nothing from it;
 * such callers can pass KEYS_FUSED or split the batch).  Both flags set:
 * LAZYATTN_EINVAL.  The two routes give the same result up to rounding; other
 * encodings, FP8 pools, framed batches and the decode ignore both flags. */
#define LAZYATTN_FLAG_KEYS_FUSED 2
#define LAZYATTN_FLAG_KEYS_ONCE 4
#define LAZYATTN_KEYS_ONCE_TILES 8

/* Pool formats (lazyattn_config.kv_format).
 *
 * PLAIN: pools hold cfg->dtype values, K [num_blocks][Hkv][16][D] and
 * V [num_blocks][Hkv][D][16].
 *
 * FP8_E4M3 (dtype bf16, D = 128 only): each (block, KV head) is one chunk of
 * LAZYATTN_FP8_CHUNK_BYTES bytes in each pool, pools [num_blocks][Hkv][chunk]:
 *   K chunk: codes [16 rows][128 channels], then int8 exponents [16], one per row;
 *   V chunk: codes [128 channels][16 tokens], then int8 exponents [16], one per token.
 * A value is its OCP e4m3 code (bias 7, largest 448) times 2^exponent.  Rows
 * are quantised whole when appended (lazyattn_append_kv): exponent = the
 * smallest e with max|x| <= 448 * 2^e (0 for an all-zero row), code = x * 2^-e
 * rounded to nearest even, saturated at +-448.  Power-of-two scales make the
 * bf16 values the kernels compute with exact.  (The pages do not describe a
 * narrower pool; this one halves the bytes a decode step streams.) */
typedef enum { LAZYATTN_KV_PLAIN = 0, LAZYATTN_KV_FP8_E4M3 = 1 } lazyattn_kv_format;
#define LAZYATTN_FP8_CHUNK_BYTES 2064

typedef struct {
  int32_t num_q_heads;    /* Hq >= 1 */
  int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;       /* D: 128 for bf16; 64 or 128 for f32 */
  int32_t block_size;     /* B: 16 */
  int32_t dtype;          /* lazyattn_dtype: queries, pools and outputs share it */
  int32_t pe;             /* lazyattn_pe */
  double rope_theta;      /* RoPE base (> 0 when pe == ROPE) */
  float softmax_scale;    /* 0 => 1/sqrt(head_dim) */
  int32_t flags;          /* LAZYATTN_FLAG_* bits; other bits must be 0 */
  const float* alibi_slopes;  /* device [Hq], or NULL => 2^(-8(h+1)/Hq) */
  const double* rope_inv_freq; /* host [head_dim/2]: angular frequency (radians per position) of
                                * channel pair i, or NULL => rope_theta^(-2i/head_dim).  Each value
                                * finite and >= 0; a 0 leaves its pair unrotated (partial rotary).
                                * Read during the call only; rope_theta is then not used.  RoPE
                                * variants: gist.science, Key Contributions > Generalizability. */
  int32_t kv_format;           /* lazyattn_kv_format */
} lazyattn_config;

/* Key frames.  With frame_starts == NULL the pool holds content-only keys
 * (gist.science, Technical Summary > Methodology: purely content-based cache)
 * and the kernels rotate every key row by R(t - p).  With frame_starts set,
 * the pool holds keys in document-local frames: the key of entry e's row at
 * logical position t is stored as R(t - F) k with F = frame_starts[r][e]
 * (a document's first position; LAZYATTN_FLAG_* unchanged), written with
 * lazyattn_append_kv_framed.  A block stays reusable at any offset, and the
 * kernels need one rotation R(F - p) per (query, frame) instead of one per key
 * (gist.science, Technical Implementation > Decoding: the query is rotated
 * only when the offset changes; > Prefilling: one relative rotation per key
 * tile).  pe ROPE and dtype bf16 (plain or FP8 pool); other configs return
 * LAZYATTN_EUNSUPPORTED when frame_starts is set. */
typedef struct {
  int32_t num_reqs;                /* R >= 0 */
  int32_t max_entries;             /* row stride of block_tables, >= every num_entries[r] */
  const uint64_t* block_tables;    /* device [R][max_entries] packed words */
  const int32_t* num_entries;      /* device [R] entries in use */
  const int32_t* ctx_lens;         /* device [R] context length L_r, this call's new tokens included */
  const int32_t* frame_starts;     /* device [R][max_entries] or NULL (content-only pool) */
  const int32_t* req_order;        /* device [R], a permutation of 0..R-1, or NULL (batch order):
                                      the order in which prefill and decode work-groups take the
                                      requests.  Results do not depend on it; longest context
                                      first shortens the tail of a batch of unequal requests.  An
                                      entry outside 0..R-1 stands for its own index; a list that is
                                      no permutation leaves some rows unwritten.  The shared-run
                                      decode ignores it. */
} lazyattn_batch;

/* ---- host-only helpers (no GPU needed) ---------------------------------- */

/* Interface version; equals LAZYATTN_ABI_VERSION of the built library. */
int32_t lazyattn_abi_version(void);

/* RoPE frequency tables for lazyattn_config.rope_inv_freq (host, out [head_dim/2]).
 *
 * lazyattn_rope_inv_freq: partial rotary.  Pair i < rotary_dim/2 gets
 * theta^(-2i/rotary_dim), the remaining pairs 0 (unrotated).  rotary_dim even,
 * 2 <= rotary_dim <= head_dim; rotary_dim == head_dim is plain RoPE.
 *
 * lazyattn_rope_inv_freq_llama31: the frequency rescaling published with the
 * Llama 3.1 models.  Base frequency f_i = theta^(-2i/head_dim) with wavelength
 * w = 2 pi / f_i: kept if w < original_max_position / high_freq_factor,
 * divided by factor if w > original_max_position / low_freq_factor, and in
 * between blended linearly in s = (original_max_position / w - low) /
 * (high - low) from f_i / factor (s = 0) to f_i (s = 1).  Requires factor >= 1,
 * 0 < low_freq_factor < high_freq_factor, original_max_position >= 1.
 *
 * Both return LAZYATTN_EINVAL on a null out or out-of-range argument. */
lazyattn_status lazyattn_rope_inv_freq(int32_t head_dim, int32_t rotary_dim, double theta, double* out);
lazyattn_status lazyattn_rope_inv_freq_llama31(int32_t head_dim, double theta, double factor, double low_freq_factor,
                                               double high_freq_factor, int32_t original_max_position, double* out);

/* Static string naming a status; never NULL. */
const char* lazyattn_status_string(lazyattn_status s);

/* Table word codec (gist.science, Technical Implementation > Decoding: block
 * id and offset bit-packed in one register).  pack = (start << 32) | block. */
uint64_t lazyattn_pack(uint32_t block_id, uint32_t logical_start);
uint32_t lazyattn_entry_block(uint64_t word);
uint32_t lazyattn_entry_start(uint64_t word);

/* Pack n host entries: words[i] = lazyattn_pack(blocks[i], starts[i]).
 * All pointers host; EINVAL if any is NULL with n > 0 or n < 0. */
lazyattn_status lazyattn_pack_entries(const uint32_t* blocks, const uint32_t* starts, int64_t n,
                                      uint64_t* words);

/* Check host copies of a batch's tables against the dense contract above and
 * against num_blocks.  On EINVAL, *bad_req and *bad_entry (host, may be NULL)
 * name the first offending request and entry (entry -1: the request's
 * num_entries/ctx_len themselves).  Reads host memory only. */
lazyattn_status lazyattn_validate_tables(const lazyattn_config* cfg, const uint64_t* tables_h,
                                         int32_t num_reqs, int32_t max_entries,
                                         const int32_t* num_entries_h, const int32_t* ctx_lens_h,
                                         int64_t num_blocks, int32_t* bad_req, int32_t* bad_entry);

/* Number of key splits a call with num_splits == 0 would use. */
int32_t lazyattn_prefill_splits(const lazyattn_config* cfg, int32_t num_reqs, int32_t max_q_len,
                                int32_t max_entries);
/* Split count for a prefill call whose table lengths the caller knows on the
 * host (max_entries = the longest request's num_entries, total_entries = their
 * sum over the batch's requests): at least lazyattn_prefill_splits(), and
 * ceil(longest / mean - 0.1), enough that the longest request's share of keys
 * per work-group is about the mean request's, so that a batch of unequal
 * lengths does not wait on its longest request; at most one split per 64
 * entries of the longest request, and at most 64.  Pass the result as
 * num_splits (and to the workspace size).  Returns 0 for an invalid config. */
int32_t lazyattn_prefill_splits_balanced(const lazyattn_config* cfg, int32_t num_reqs, int32_t max_q_len,
                                         int32_t max_entries, int64_t total_entries);
int32_t lazyattn_decode_splits(const lazyattn_config* cfg, int32_t num_reqs, int32_t max_entries);

/* Workspace bytes for a prefill/decode call with these sizes (num_splits as
 * passed to the call; 0 => the heuristic).  0 means no workspace needed.
 * A call that splits the key range into S > 1 parts writes partial results
 * to the workspace: each part's output already divided by its own softmax
 * sum, as IEEE half, o [S][rows][Hq][D], then its reference and sum (m, l)
 * as fp32 [S][rows][Hq][2] (rows = total_q for prefill, num_reqs for
 * decode), S*rows*Hq*(2D + 8) bytes; the merge kernel then combines them.
 * Range: each split's output is a convex combination of value rows, stored as
 * IEEE half, so a call with S > 1 requires |v| <= 65504 for every value it
 * reads (a larger value overflows its partial and the merged output is not
 * finite); with S = 1 the output is written as bf16 directly and no such limit
 * applies.  A prefill call that turns the keys once (LAZYATTN_FLAG_KEYS_ONCE,
 * or the library's choice without a flag) also holds the turned keys there,
 * after the partials rounded up to 256 bytes: bf16 [num_reqs][Hkv][max_entries]
 * chunks of [16][D] (request r's entry e for KV head h at chunk
 * (r * Hkv + h) * max_entries + e), num_reqs * max_entries * Hkv * 4096 bytes; the
 * size counts them whenever the route would be taken for these sizes (a framed
 * batch, which does not take it, needs less).  The workspace needs no
 * initialisation; calls that may run concurrently must not share one. */
size_t lazyattn_prefill_workspace_size(const lazyattn_config* cfg, int32_t num_reqs, int32_t total_q,
                                       int32_t max_q_len, int32_t max_entries, int32_t num_splits);
size_t lazyattn_decode_workspace_size(const lazyattn_config* cfg, int32_t num_reqs,
                                      int32_t max_entries, int32_t num_splits);

/* ---- GPU entry points ---------------------------------------------------- */

/* Causal prefill of each request's new tokens over its whole context
 * (gist.science, Technical Implementation > Prefilling: the kernel loads KV
 * blocks from the cache and applies one relative rotation per key tile).
 *  q          device [total_q][Hq][D]; request r owns rows
 *             cu_q_lens[r] .. cu_q_lens[r+1]-1 and its j-th row sits at
 *             logical position ctx_lens[r] - q_len_r + j.  The new tokens'
 *             K/V must already be in the pool (lazyattn_append_kv).
 *  cu_q_lens  device [R+1] int32 prefix sums, cu_q_lens[0] = 0
 *  total_q    host, = cu_q_lens[R]; max_q_len host, >= every q_len_r
 *  k_pool, v_pool device pools of num_blocks blocks
 *  batch      host struct holding device arrays
 *  num_splits 0 => heuristic; else 1..64 splits of the key range
 *  out        device [total_q][Hq][D]
 *  workspace  device, >= lazyattn_prefill_workspace_size(...) bytes (may be
 *             NULL when that size is 0).
 *  Launches the key-turning kernel when the keys are turned once (see
 *  LAZYATTN_FLAG_KEYS_ONCE), the attention kernel and, when the key range is
 *  split, the merge kernel (lazyattn_prefill_attend followed by
 *  lazyattn_merge_splits). */
lazyattn_status lazyattn_prefill(const lazyattn_config* cfg, const void* q, const int32_t* cu_q_lens,
                                 int32_t total_q, int32_t max_q_len, const void* k_pool,
                                 const void* v_pool, int64_t num_blocks, const lazyattn_batch* batch,
                                 int32_t num_splits, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* One decode step (gist.science, Technical Implementation > Decoding): request
 * r's single query q[r] sits at position ctx_lens[r]-1 and its own K/V is
 * already in the pool.
 *  q    device [R][Hq][D];  out device [R][Hq][D]
 *  num_splits 0 => heuristic; else 1..256 splits of each request's entries
 *  workspace as for prefill (>= lazyattn_decode_workspace_size bytes).
 *  Launches the attention kernel and, when split, the merge kernel.  bf16
 *  supports G = Hq/Hkv <= 32. */
lazyattn_status lazyattn_decode(const lazyattn_config* cfg, const void* q, const void* k_pool,
                                const void* v_pool, int64_t num_blocks, const lazyattn_batch* batch,
                                int32_t num_splits, void* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* lazyattn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels and results, with the split partials written to a device
 * array the library owns (LAZYATTN_DECODE_SCRATCH_BYTES per GPU, held from the
 * first call on that GPU until the process ends) instead of a workspace
 * argument.  The caller still passes q and out.  Makes no allocation.
 *  - Returns LAZYATTN_EWORKSPACE, before any launch, when the call's split
 *    partials (lazyattn_decode_workspace_size with the same arguments) exceed
 *    LAZYATTN_DECODE_SCRATCH_BYTES; pass a smaller num_splits, or use
 *    lazyattn_decode with a workspace.
 *  - Every call on one GPU shares that GPU's array: calls that may overlap on
 *    one GPU (several streams, several threads) race and must not be issued.
 *    Nothing in it needs clearing between calls (each call writes every
 *    partial it reads).
 *  - The first call on a device looks up the array's device address there.
 * Other arguments and errors as lazyattn_decode. */
#define LAZYATTN_DECODE_SCRATCH_BYTES (16u << 20)
lazyattn_status lazyattn_decode_noalloc(const lazyattn_config* cfg, const void* q, const void* k_pool,
                                        const void* v_pool, int64_t num_blocks, const lazyattn_batch* batch,
                                        int32_t num_splits, void* out, hipStream_t stream);

/* ---- decode over shared runs ----------------------------------------------
 * A pool block holds content only, so one physical copy of a document serves
 * every request that holds it, at whatever position (gist.science, Technical
 * Summary > Methodology: purely content-based cache; shd-paper.top, Abstract:
 * one physical KV copy shared by many logical requests).  lazyattn_decode
 * reads such a block once per request that holds it; these two calls read it
 * about once per batch.
 *
 * lazyattn_decode_runs_plan (host) cuts the tables into runs: maximal
 * sequences of entries, (block, valid length) each, that follow one another in
 * the same order wherever they occur (typically a shared document); all but a
 * run's last entry are whole blocks.  Every entry of every request lies in
 * exactly one occurrence of one run.  A run held more than once is cut into
 * work items of at most 64 entries and at most 16 / G occurrences (G =
 * Hq / Hkv; the query rows of one 16-row MFMA tile), listed so that
 * round-robin dispatch puts the items of one run piece on one XCD, where their
 * reads of the same blocks meet in its L2.  The entries of runs held once are
 * gathered per request into items of at most 128 entries and one occurrence.
 *
 * lazyattn_decode_runs attends each item once per KV head, one wave per item
 * (items 4 m .. 4 m + 3 form work-group m).  An item's entries
 * carry key offsets o from a base s of the item (a shared run's first key; 0
 * for a request's own entries), and each occurrence an offset p - s, p the
 * request's query position: the key rows are turned by R(o) and the query of
 * each occurrence by R(p - s).  Since R(t - p) = R(o) R(s - p) for the key at
 * t = s + o, the scores are the per-request ones (gist.science, Technical
 * Summary > Mathematical Equivalence).  Each occurrence and head gets a
 * partial (o / l in fp16, m, l), and a second kernel merges each request's
 * partials by log-sum-exp in occurrence order.  Results equal
 * lazyattn_decode's up to rounding (the query is rounded to bf16 after its
 * turn; the summation order differs).  The partials are IEEE half, so every
 * value must satisfy |v| <= 65504, as for a split lazyattn_decode call. */
#define LAZYATTN_RUN_ITEM_INTS 4
typedef struct {
  int32_t num_items;              /* work items; a multiple of 32, padded with empty items */
  int32_t num_words;              /* item entries */
  int32_t num_refs;               /* occurrences over all items = partial slots */
  const int32_t* items;           /* device [num_items][LAZYATTN_RUN_ITEM_INTS]: {first word,
                                     entries (0: an empty item), first occurrence, occurrences} */
  const uint64_t* words;          /* device [num_words] item entries: physical block in bits
                                     31..0, key offset o in bits 58..32, valid length in 63..59 */
  const int32_t* refs;            /* device [num_refs][2] {request, p - s} */
  const int32_t* req_ref_begin;   /* device [R + 1]: request r's occurrences are */
  const int32_t* req_refs;        /* device [num_refs]: req_refs[req_ref_begin[r] .. req_ref_begin[r+1]) */
} lazyattn_run_plan;

/* Build the plan on the host from host copies of a decode batch's tables
 * (the layout of lazyattn_batch; tables are checked as by
 * lazyattn_validate_tables, EINVAL on a violation).  Writes the needed sizes
 * to *num_items, *num_words and *num_refs in every case (with zero
 * capacities, that is all it does) and fills the host arrays
 *  items_h [capacity_items][LAZYATTN_RUN_ITEM_INTS], words_h [capacity_words],
 *  refs_h [capacity_refs][2], req_ref_begin_h [num_reqs + 1], req_refs_h [capacity_refs]
 * only when every capacity suffices (else LAZYATTN_EWORKSPACE, arrays
 * untouched); the caller copies them to the device for lazyattn_decode_runs.
 * The plan depends on the tables only, not on the pool's contents.
 * LAZYATTN_EUNSUPPORTED unless dtype is bf16 and G <= 16, and for a request
 * entry starting at 2^27 or later.  A request with no
 * entries has no occurrence; its output rows become zero. */
lazyattn_status lazyattn_decode_runs_plan(const lazyattn_config* cfg, const uint64_t* tables_h, int32_t num_reqs,
                                          int32_t max_entries, const int32_t* num_entries_h,
                                          const int32_t* ctx_lens_h, int64_t num_blocks, int32_t capacity_items,
                                          int32_t capacity_words, int32_t capacity_refs, int32_t* items_h,
                                          uint64_t* words_h, int32_t* refs_h, int32_t* req_ref_begin_h,
                                          int32_t* req_refs_h, int32_t* num_items, int32_t* num_words,
                                          int32_t* num_refs);

/* Bytes of workspace lazyattn_decode_runs needs: the partials of num_refs
 * occurrences; 0 for an invalid config. */
size_t lazyattn_decode_runs_workspace_size(const lazyattn_config* cfg, int32_t num_refs);

/* One decode step over a plan (see above): q, out device [num_reqs][Hq][D] as
 * for lazyattn_decode, the pool content-only (plain or FP8), workspace >=
 * lazyattn_decode_runs_workspace_size bytes.  Launches the attention kernel
 * (num_items x Hkv work-groups) and the merge kernel on `stream`.  The plan's
 * arrays must describe this batch: an item or occurrence outside the pool or
 * the batch is not detected here (lazyattn_decode_runs_plan builds valid ones).
 * EUNSUPPORTED as for the plan; EWORKSPACE for a short workspace. */
lazyattn_status lazyattn_decode_runs(const lazyattn_config* cfg, const void* q, const void* k_pool,
                                     const void* v_pool, int64_t num_blocks, int32_t num_reqs,
                                     const lazyattn_run_plan* plan, void* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* The attention kernel of lazyattn_prefill / lazyattn_decode alone (same
 * arguments; for a prefill that turns the keys once, the key-turning kernel
 * and then the attention kernel).  With one split it writes `out` directly; with S > 1 splits
 * (see lazyattn_prefill_splits / lazyattn_decode_splits for num_splits 0) it
 * writes partials to `workspace` and leaves `out` untouched until
 * lazyattn_merge_splits runs on the same stream.  For callers that schedule
 * or time the two kernels separately. */
lazyattn_status lazyattn_prefill_attend(const lazyattn_config* cfg, const void* q, const int32_t* cu_q_lens,
                                        int32_t total_q, int32_t max_q_len, const void* k_pool,
                                        const void* v_pool, int64_t num_blocks, const lazyattn_batch* batch,
                                        int32_t num_splits, void* out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);
lazyattn_status lazyattn_decode_attend(const lazyattn_config* cfg, const void* q, const void* k_pool,
                                       const void* v_pool, int64_t num_blocks, const lazyattn_batch* batch,
                                       int32_t num_splits, void* out, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* Log-sum-exp merge of S split partials into out [num_rows][Hq][D] (bf16):
 * with w_s = 2^(m_s - M) l_s and M = max_s m_s, out = sum_s w_s o_s / sum_s w_s
 * (o_s already divided by l_s), summed in split order.  num_rows = total_q
 * (prefill) or num_reqs (decode); workspace as written by the matching
 * *_attend call with S = num_splits.  num_splits 1 is a no-op.  EWORKSPACE if
 * workspace_bytes is short of S*num_rows*Hq*(2D+8). */
lazyattn_status lazyattn_merge_splits(const lazyattn_config* cfg, int32_t num_rows, int32_t num_splits,
                                      const void* workspace, size_t workspace_bytes, void* out,
                                      hipStream_t stream);

/* Write n new tokens' content-only K/V into the pool (gist.science,
 * Methodology: the cache stores content-based keys and values, no rotation).
 *  k_new, v_new device [n][Hkv][D] in cfg->dtype; slots device [n] int64 =
 *  block*B + row, every slot < num_blocks*B (not checked on the device).
 *  FP8 pool format: k_new/v_new are bf16 and each row is quantised as
 *  "Pool formats" describes (the row's exponent is written with it). */
lazyattn_status lazyattn_append_kv(const lazyattn_config* cfg, void* k_pool, void* v_pool,
                                   int64_t num_blocks, const void* k_new, const void* v_new,
                                   const int64_t* slots, int32_t n, hipStream_t stream);

/* ---- materialise-then-attend baseline (for comparison only) -------------
 * The approach deferred positional encoding replaces: existing systems give
 * each request its own copy of a cached document with positions re-encoded,
 * paying memory and bandwidth for the copy (shd-paper.top digest, original
 * abstract; gist.science, Technical Summary > Problem Statement).  These two
 * calls build that copy so its cost can be measured next to the deferred
 * kernels: materialise the KV, rotate the queries, then run lazyattn_prefill
 * with pe = NONE on the copy (same result up to rounding, since
 * R(p)^T R(t) = R(t - p)).  bf16, D = 128, pe ROPE, plain content-only pools
 * only (frame_starts set or an FP8 format: LAZYATTN_EUNSUPPORTED). */

/* Copy every entry of every request from the shared pool into the private
 * block that dst_tables names at the same (request, entry), K rows rotated by
 * R(t) at their logical position t = start + row, V unchanged.
 *  batch       the source tables (device), as for prefill
 *  dst_tables  device [R][batch->max_entries] packed words; only the block ids
 *              are used, each < dst_num_blocks and written by one entry only
 *  dst_k_pool, dst_v_pool  device pools of dst_num_blocks blocks, same layout
 *              as the source pools; the source pools are only read.
 *  Rows past an entry's length are copied as they are. */
lazyattn_status lazyattn_materialize_kv(const lazyattn_config* cfg, const void* k_pool, const void* v_pool,
                                        int64_t num_blocks, const lazyattn_batch* batch,
                                        const uint64_t* dst_tables, void* dst_k_pool, void* dst_v_pool,
                                        int64_t dst_num_blocks, hipStream_t stream);

/* Rotate every query row by R(p) at its logical position p (laid out and
 * positioned as for lazyattn_prefill) into q_out device [total_q][Hq][D]. */
lazyattn_status lazyattn_rotate_queries(const lazyattn_config* cfg, const void* q, const int32_t* cu_q_lens,
                                        int32_t total_q, int32_t max_q_len, const lazyattn_batch* batch,
                                        void* q_out, hipStream_t stream);

/* lazyattn_append_kv for a pool in document-local frames: token i's key is
 * stored as R(frame_index[i]) k_new[i] (frame_index = its logical position
 * minus its frame's start), its value unchanged.  frame_index device [n]
 * int32.  pe ROPE, bf16 only; with the FP8 pool format the key is turned in
 * float and then quantised. */
lazyattn_status lazyattn_append_kv_framed(const lazyattn_config* cfg, void* k_pool, void* v_pool,
                                          int64_t num_blocks, const void* k_new, const void* v_new,
                                          const int64_t* slots, const int32_t* frame_index, int32_t n,
                                          hipStream_t stream);

/* Decode every table entry on the device exactly as the attention kernels do
 * and write (block id, logical start, valid length) as int32 triples to
 * out [R][max_entries][3] (device); entries >= num_entries[r] get (-1,-1,-1). */
lazyattn_status lazyattn_debug_decode_tables(const lazyattn_batch* batch, int32_t* out,
                                             hipStream_t stream);

/* ---- block pool manager (host only) ----------------------------------------
 *
 * Which physical blocks hold which cached document, under a fixed block
 * budget with least-recently-used eviction.  The cache key is the policy's:
 *   POSITION_AGNOSTIC  the document alone: one copy serves every offset (the
 *                      content-only pool the kernels above read);
 *   POSITION_AWARE     (document, logical start): a document cached at one
 *                      offset is a miss at any other, and each offset keeps its
 *                      own copy;
 *   PREFIX             the chain of documents up to and including this one: a
 *                      document hits only if every earlier document of the
 *                      request hit and the whole chain was cached before.
 * (gist.science, Technical Summary > Problem Statement: position-aware caches
 * hold several variants of one document and prefix reuse needs identical
 * prefixes, which lowers the hit ratio under skewed access; > Key
 * Contributions and > Experimental Results report the hit ratios.)
 *
 * A request is admitted whole: its documents in context order, document k at
 * logical start sum(len[0..k-1]).  A miss allocates ceil(len / 16) blocks,
 * evicting unpinned entries from the least recently used end while blocks are
 * short; if they stay short, the document is bypassed (not cached, no blocks).
 * Every cached document of an admitted request stays pinned (never evicted)
 * until the request is released; on release its documents become the most
 * recently used, in context order.  A PREFIX-policy document found cached
 * after an earlier miss of the same request counts as a miss (its keys would
 * be recomputed) and reuses its entry.  Not thread-safe: one caller per pool. */
typedef enum {
  LAZYATTN_CACHE_POSITION_AGNOSTIC = 0,
  LAZYATTN_CACHE_POSITION_AWARE = 1,
  LAZYATTN_CACHE_PREFIX = 2
} lazyattn_cache_policy;

typedef struct lazyattn_pool lazyattn_pool;   /* opaque */

typedef struct {
  int64_t num_blocks;       /* the budget */
  int64_t blocks_in_use;    /* held by cached documents */
  int64_t doc_accesses, doc_hits;
  int64_t token_accesses, token_hits;
  int64_t inserts, evictions, bypasses;
  int64_t open_requests;    /* admitted, not yet released */
} lazyattn_pool_stats;

/* Document admission outcome (doc_status of lazyattn_pool_admit). */
#define LAZYATTN_DOC_MISS 0    /* blocks newly assigned: the caller writes the document's K/V into them */
#define LAZYATTN_DOC_HIT 1     /* the cached copy is used as is */
#define LAZYATTN_DOC_BYPASS 2  /* no blocks: the budget is held by pinned documents */

/* Create a pool of num_blocks >= 0 blocks (ids 0..num_blocks-1) with the
 * given policy; *out receives the handle (freed by lazyattn_pool_destroy).
 * EINVAL on a bad policy or size. */
lazyattn_status lazyattn_pool_create(int64_t num_blocks, int32_t policy, lazyattn_pool** out);
void lazyattn_pool_destroy(lazyattn_pool* pool);

/* Admit one request of n_docs documents (doc_ids [n_docs] >= 0, doc_lens
 * [n_docs] >= 1, host arrays).  Writes doc_status [n_docs] and, for every
 * document that is not bypassed, its table entries in context order:
 * blocks [*num_entries] and starts [*num_entries] (logical start of each
 * block, as lazyattn_pack_entries takes them), at most max_entries of them.
 * *ticket identifies the request for lazyattn_pool_release.  EINVAL on bad
 * arguments; EWORKSPACE if the entries do not fit max_entries (the pool is
 * then unchanged). */
lazyattn_status lazyattn_pool_admit(lazyattn_pool* pool, const int64_t* doc_ids, const int32_t* doc_lens,
                                    int32_t n_docs, uint32_t* blocks, uint32_t* starts, int32_t max_entries,
                                    int32_t* num_entries, uint8_t* doc_status, int64_t* ticket);

/* Unpin the documents of an admitted request.  EINVAL on an unknown ticket. */
lazyattn_status lazyattn_pool_release(lazyattn_pool* pool, int64_t ticket);

lazyattn_status lazyattn_pool_get_stats(const lazyattn_pool* pool, lazyattn_pool_stats* out);

/* Admit and release n_requests requests in order: request i holds documents
 * req_offsets[i] .. req_offsets[i+1]-1 of doc_ids / doc_lens (host arrays).
 * The statistics accumulate in the pool.  EINVAL on bad arguments. */
lazyattn_status lazyattn_pool_run_trace(lazyattn_pool* pool, const int64_t* doc_ids, const int32_t* doc_lens,
                                        const int64_t* req_offsets, int64_t n_requests);

#ifdef __cplusplus
}
#endif

#endif /* LAZYATTN_H */
