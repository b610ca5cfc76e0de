/*
 * pkv.h - C ABI of libpkv, paged GQA decode attention for MI355X (gfx950).
 *
 * One decode step of a transformer layer: every sequence in the batch has one
 * new token whose query attends over that sequence's cached keys and values,
 * softmax(q K^T * scale) V, with K/V stored in fixed-size pages found through a
 * per-sequence block table and each KV head shared by a group of query heads.
 *
 * Sources for the operations (web pages on LLM inference):
 *  - attention and the cache it forces: evaltude "Part 6 - Inference
 *    Fundamentals", section "Q, K, V - and why they force a cache"; evaltude
 *    docs "Transformer inference mechanics", sections "What Q, K, and V do in
 *    causal attention" and "What the KV cache stores per layer";
 *  - MHA / MQA / GQA head sharing: the same docs, "MHA versus MQA versus GQA";
 *  - paged storage, 16-token blocks, per-request block table: hoshank.vercel.app
 *    "Inference Engines" (chapter 17), "The Breakthrough"; CS336 lecture 10
 *    notes (rraushan-blog), "PagedAttention (vLLM)";
 *  - online softmax, exact rescaling of partial results: learn.byteknotlabs.com
 *    "Efficient inference", "FlashAttention: exact attention without the
 *    matrix"; split-KV decode (FlashDecoding) is named in the CS336 notes;
 *  - KV byte formula: chapter 17 "The Mathematics" (equation M_kv).
 *
 * Conventions
 *  - Every function returns an int status (PKV_OK = 0 or a negative PKV_ERR_*)
 *    unless stated otherwise; no C++ exception crosses the ABI.  On error,
 *    pkv_last_error() returns a thread-local description.
 *  - "device" pointers are HIP device memory owned by the caller; the library
 *    never allocates, frees or synchronises device memory and launches only on
 *    the given stream (a hipStream_t passed as void*, NULL = default stream).
 *    Device calls return after the launch (asynchronous); a launch failure
 *    returns PKV_ERR_HIP.
 *  - "host" pointers are ordinary CPU memory owned by the caller.
 *  - All scalar arguments are checked on the host before anything is
 *    launched; nothing is launched on error.  Device-side data (block-table
 *    entries, lengths, positions) is checked in the kernels: an entry that
 *    would address outside the pool is never dereferenced (see each call).
 *
 * Data layout (device, row-major; elem = float or bfloat16; X = 16 / sizeof(elem),
 * i.e. 4 for fp32 and 8 for bf16; the block size is 16 tokens):
 *  - q        [batch][n_q_heads][head_dim]
 *  - out      [batch][n_q_heads][head_dim] (same dtype as q)
 *  - k_pages  [num_pages][n_kv_heads][head_dim / X][16][X]: key element d of the
 *             token in slot s of page p, head h, is at [p][h][d / X][s][d % X];
 *  - v_pages  [num_pages][n_kv_heads][head_dim][16]: value element d of slot s
 *             is at [p][h][d][s] (V is stored transposed inside a page);
 *  - block_table int32 [batch][max_blocks_per_seq]: logical block i of sequence
 *             b lives in physical page block_table[b][i]; entries past the
 *             sequence's last block are ignored (-1 by convention);
 *  - seq_lens int32 [batch]: number of tokens each query attends to, all of
 *             them already in the cache (token t < seq_len is slot t % 16 of
 *             page block_table[b][t / 16]).
 *  - GQA head map: query head hq reads KV head hq / (n_q_heads / n_kv_heads).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size or shape   */
  PKV_ERR_UNSUPPORTED = -2,  /* valid but not built: head_dim, dtype, block  */
  PKV_ERR_OUT_OF_PAGES = -3, /* pool exhausted; the pool is left unchanged   */
  PKV_ERR_WORKSPACE = -4,    /* workspace smaller than required              */
  PKV_ERR_HIP = -5,          /* a HIP runtime call or launch failed          */
  PKV_ERR_NOT_FOUND = -6,    /* unknown sequence id                          */
  PKV_ERR_EXISTS = -7        /* sequence id already in use                   */
};

/* Element types.  PKV_U8 names the 8-bit KV cache below (its q and out are
 * bf16); the dense calls take PKV_F32 or PKV_BF16. */
enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_U8 = 2 };

/* Description of a status code (static string). */
const char* pkv_status_string(int status);
/* Detail of the last error on the calling thread ("" if none). */
const char* pkv_last_error(void);
/* Library version string, e.g. "pkv 0.1.0 gfx950". */
const char* pkv_version(void);

/* ------------------------------------------------------------------------ *
 * Byte accounting (host).  Chapter 17 "The Mathematics", equation M_kv:
 *   M = 2 * n_layers * n_kv_heads * head_dim * seq_len * batch * elem_bytes
 * (factor 2: keys and values).  Returns 0 if any argument is negative.
 * ------------------------------------------------------------------------ */
uint64_t pkv_kv_cache_bytes(int64_t n_layers, int64_t n_kv_heads, int64_t head_dim,
                            int64_t seq_len, int64_t batch, int64_t elem_bytes);
/* Per-token form (seq_len = batch = 1). */
uint64_t pkv_kv_bytes_per_token(int64_t n_layers, int64_t n_kv_heads, int64_t head_dim,
                                int64_t elem_bytes);

/* ------------------------------------------------------------------------ *
 * Page pool and block tables (host).  Blocks are allocated on demand as a
 * sequence grows, from a free list, instead of reserving a worst-case slab
 * (chapter 17 "The Breakthrough"; CS336 notes "PagedAttention (vLLM)").
 * Rules:
 *  - the free list starts in the order given (free_order: a permutation of
 *    0..num_pages-1; NULL means 0, 1, 2, ...);
 *  - reserve takes pages from the front of the free list, in order;
 *  - release returns a sequence's pages, in block order, to the back of the
 *    free list (a page shared by a fork is returned when its last user goes);
 *  - fork lets a child share all of a parent's pages (reference counted);
 *    reserve_for_write replaces a shared block with a fresh page before a
 *    write (copy-on-write, CS336 notes "PagedAttention (vLLM)").
 * A pool is not thread-safe; use one per thread or lock around calls.
 * ------------------------------------------------------------------------ */
typedef struct pkv_pool pkv_pool;

/* Create a pool of num_pages (>= 1) pages.  *out receives the pool. */
int pkv_pool_create(int32_t num_pages, const int32_t* free_order /* host, nullable */,
                    pkv_pool** out);
void pkv_pool_destroy(pkv_pool* pool);
/* Number of free pages, or a negative status if pool is NULL. */
int32_t pkv_pool_num_free(const pkv_pool* pool);
/* Grow seq_id (created if new) to hold n_tokens tokens, i.e. ceil(n_tokens /
 * block_size) blocks.  Never shrinks.  *n_new_pages (nullable) receives the
 * number of pages taken.  PKV_ERR_OUT_OF_PAGES leaves the pool unchanged. */
int pkv_seq_reserve(pkv_pool* pool, int64_t seq_id, int64_t n_tokens, int32_t block_size,
                    int32_t* n_new_pages);
/* Forget seq_id and return its pages (PKV_ERR_NOT_FOUND if unknown). */
int pkv_seq_release(pkv_pool* pool, int64_t seq_id);
/* child shares every page of parent (PKV_ERR_EXISTS if child exists). */
int pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t child);
/* Make token `position` of seq_id writable: grow it if needed; if the block
 * holding position is shared, give seq_id a fresh page for it.  *copy_src and
 * *copy_dst receive (old page, new page) when the caller must copy the block's
 * contents, or -1 and -1 when no copy is needed. */
int pkv_seq_reserve_for_write(pkv_pool* pool, int64_t seq_id, int64_t position,
                              int32_t block_size, int32_t* copy_src, int32_t* copy_dst);
/* Number of blocks held by seq_id. */
int pkv_seq_num_blocks(const pkv_pool* pool, int64_t seq_id, int32_t* out);
/* Fill out (host int32 [batch][max_blocks_per_seq]) with each sequence's pages
 * in logical order, padded with -1.  Unknown ids give an all -1 row.  Returns
 * PKV_ERR_INVALID_ARG if a sequence has more than max_blocks_per_seq blocks. */
int pkv_build_block_table(const pkv_pool* pool, const int64_t* seq_ids, int32_t batch,
                          int32_t max_blocks_per_seq, int32_t* out);

/* ------------------------------------------------------------------------ *
 * kv_append (device): write the step's new key and value of every sequence
 * into its slot (evaltude docs "What the KV cache stores per layer": each
 * layer's cache gains the new token's K/V every step).
 *   k_new, v_new  device [batch][n_kv_heads][head_dim] (dtype)
 *   positions     device int32 [batch]: token index to write; it lands in slot
 *                 positions[b] % 16 of page block_table[b][positions[b] / 16].
 * A bit-for-bit copy.  A position < 0 or >= 16 * max_blocks_per_seq, or a
 * block-table entry outside [0, num_pages), skips that sequence's write (no
 * memory outside the pool is touched).
 * ------------------------------------------------------------------------ */
int pkv_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                  const int32_t* block_table, const int32_t* positions, int32_t batch,
                  int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t max_blocks_per_seq, int32_t num_pages, int32_t dtype, void* stream);

/* ------------------------------------------------------------------------ *
 * paged_decode_attn (device): out[b][hq] = softmax(scale * q[b][hq] . K_b^T) V_b
 * over the seq_lens[b] cached tokens of sequence b and KV head
 * hq / (n_q_heads / n_kv_heads), computed with an online softmax (running
 * maximum and sum, no score matrix) and split over the KV pages; the splits'
 * partial results are merged by a log-sum-exp combine.
 *
 * Supported: head_dim 64 or 128; block_size 16; dtype PKV_F32 or PKV_BF16 (q,
 * pages and out share it; accumulation is fp32); n_q_heads a multiple of
 * n_kv_heads with group n_q_heads / n_kv_heads <= 64; 0 <= batch <= 15000.
 * seq_lens[b] == 0 gives a zero row.  A length < 0 or > 16 * max_blocks_per_seq,
 * or a block-table entry outside [0, num_pages), gives a NaN row for that
 * sequence (nothing outside the pool is read).
 *
 * Work split: the pages of all (sequence, KV head) pairs, taken in that order,
 * are cut into n_items equal chunks of C = max(min_chunk_pages,
 * ceil(total / n_items)) pages.  Each chunk is processed by one wavefront per
 * block of 16 query heads of the group (1, 2 or 4 wavefronts; a 3-block group
 * uses 4, the last idle).  A (sequence, KV head)
 * whose pages fall in one chunk gets its output written directly; otherwise
 * each chunk writes a partial (normalised output and natural-log sum of
 * exponentials) and the partials are merged.  By default the chunk that
 * finishes a pair last merges them in the same launch (arrival counted by
 * one atomic per chunk; merge order is fixed, so results are run-to-run
 * identical); pairs that may span more than 96 chunks (ceil(max_blocks_per_seq
 * / min_chunk_pages) + 1 > 96) are merged by a second kernel, which is then
 * launched on the same stream.  With 33 to 64 query columns per KV head
 * (query heads per KV head times query tokens) the bound is 24 chunks, and
 * above it only pairs of at most 8 chunks are merged in the decode kernel.
 * Either way every pair is merged by the same formula in a fixed order.
 *
 * workspace: device, 256-byte aligned, at least
 * pkv_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, n_items)
 * bytes (n_items after defaults are applied).  Layout: the partials from
 * offset 0, then (256-byte aligned) 4 * (batch + 1) bytes where the split
 * kernel stores the per-sequence page prefix for the combine kernel.  The
 * counters are at the END of the workspace, counted backwards from its last
 * int32 word (word workspace_bytes / 4 - 1): that word is the dynamic
 * schedule's chunk counter, and the 4 * batch * n_kv_heads words below it
 * are the arrival counters, (b, h, head block j) at word
 * workspace_bytes / 4 - 2 - ((b * n_kv_heads + h) * 4 + j).  Their place
 * depends only on workspace_bytes, so one workspace, sized for the largest
 * batch, serves calls with any smaller batch (continuous batching).
 * Partials and prefix are overwritten by every call; the counters must be
 * zero before the first call that uses the workspace (e.g. a zero-filled
 * allocation), and every call leaves them zero.  Calls that overlap in time
 * must not share a workspace.
 * opts (nullable): n_items <= 0 means, for groups of at most 16 query heads
 * (one wavefront per chunk), one chunk per wavefront of one workgroup per CU
 * (4 x CUs), and for larger groups as many chunks as the device holds at
 * once (resident wavefronts divided by the wavefronts per chunk); under the
 * dynamic schedule, 8 chunks per wavefront of one workgroup per CU;
 * min_chunk_pages <= 0 means 64 pages (groups <= 16) or 32 (larger groups,
 * and the 8-bit cache, dtype PKV_U8, at every group size), 16 under the
 * dynamic schedule;
 * combine_mode 0 merges in the decode kernel where the bound above allows,
 * 1 always merges with the separate combine kernel (counters untouched);
 * schedule (pkv_schedule) chooses how chunks are given to wavefronts.  The
 * chunks, and so the results bit for bit, depend only on n_items and
 * min_chunk_pages, not on the schedule.  The dynamic schedule takes at most
 * 16 columns per KV head (query heads per KV head times query tokens).
 * ------------------------------------------------------------------------ */
typedef enum {
  PKV_SCHEDULE_AUTO = 0,     /* the library's choice (currently static) */
  PKV_SCHEDULE_STATIC = 1,   /* chunk i to wavefront (group) i, fixed at launch */
  PKV_SCHEDULE_DYNAMIC = 2   /* one workgroup per CU, chunks handed out as wavefronts free up */
} pkv_schedule;

typedef struct pkv_decode_opts {
  int32_t n_items;
  int32_t min_chunk_pages;
  int32_t combine_mode;
  int32_t schedule;          /* pkv_schedule */
} pkv_decode_opts;

int pkv_paged_decode_attn(const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, const int32_t* seq_lens,
                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                          int32_t block_size, float scale, void* out, void* stream,
                          int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                          int32_t dtype, void* workspace, size_t workspace_bytes,
                          const pkv_decode_opts* opts);

/* One decode step in one pass over the cache: kv_append of every sequence's
 * new token followed by paged_decode_attn, with the append done inside the
 * decode kernel.  The new token is the last attended one: sequence b's
 * k_new[b]/v_new[b] (device [batch][n_kv_heads][head_dim], dtype) are written
 * to position seq_lens[b] - 1 (slot (seq_lens[b] - 1) % 16 of page
 * block_table[b][(seq_lens[b] - 1) / 16]) and attended together with the
 * seq_lens[b] - 1 tokens already cached.  The wavefront that computes a
 * sequence's last page uses the new token from registers and stores it to
 * the pool, so the result and the pool equal pkv_kv_append with positions =
 * seq_lens - 1 followed by pkv_paged_decode_attn.  Sequences with seq_lens 0
 * append nothing; an invalid last-page id skips the store (NaN row as above).
 * Same shapes, workspace and options as pkv_paged_decode_attn. */
int pkv_decode_step(const void* q, const void* k_new, const void* v_new, void* k_pages,
                    void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                    float scale, void* out, void* stream, int32_t batch,
                    int32_t max_blocks_per_seq, int32_t num_pages, int32_t dtype, void* workspace,
                    size_t workspace_bytes, const pkv_decode_opts* opts);

/* pkv_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same call without the workspace argument.  Its workspace is a fixed
 * 16 MiB array in the library's device code (16777216 bytes, one per GPU,
 * held until the process ends); the call allocates nothing and calls no
 * allocating routine.  Shapes whose workspace (pkv_decode_resolve) exceeds
 * 16 MiB are refused with PKV_ERR_WORKSPACE before anything is launched;
 * the five workloads of this library's tests fit (the largest, a 131072-token
 * MQA layer, needs 8.5 MB).  The first call on a device also launches one
 * fill kernel on `stream` that zeroes the array.  Every call on a GPU shares
 * that GPU's array, so calls that overlap in time on one GPU race (as calls
 * sharing a workspace do): serialize them, e.g. on one stream.  Same
 * arguments, options, results and pool writes as pkv_decode_step. */
int pkv_decode_step_noalloc(const void* q, const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                            const int32_t* block_table, const int32_t* seq_lens, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, int32_t block_size, float scale, void* out,
                            void* stream, int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                            int32_t dtype, const pkv_decode_opts* opts);

/* The split half of pkv_decode_step alone (same arguments): the fused append
 * and the decode kernel, leaving multi-chunk rows to pkv_lse_combine exactly
 * as pkv_paged_decode_split does. */
int pkv_decode_step_split(const void* q, const void* k_new, const void* v_new, void* k_pages,
                          void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                          int32_t block_size, float scale, void* out, void* stream, int32_t batch,
                          int32_t max_blocks_per_seq, int32_t num_pages, int32_t dtype,
                          void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts);

/* The split half of pkv_paged_decode_attn alone (same arguments; never
 * merges, never touches the counters): writes the rows of single-chunk
 * (sequence, KV head) pairs into out and every other chunk's partial into
 * the workspace:
 *   partial_o   float [slots][group][head_dim] at workspace offset 0
 *   partial_lse float [slots][group] right after partial_o
 * with slots = n_items + batch * n_kv_heads; chunk c's partial for pair
 * (b, h) is slot c + b * n_kv_heads + h.  partial_o is softmax-weighted V over
 * the chunk's tokens of that pair, partial_lse = log(sum exp(scale * q.k)). */
int pkv_paged_decode_split(const void* q, const void* k_pages, const void* v_pages,
                           const int32_t* block_table, const int32_t* seq_lens,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           int32_t block_size, float scale, void* out, void* stream,
                           int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                           int32_t dtype, void* workspace, size_t workspace_bytes,
                           const pkv_decode_opts* opts);

/* The combine half: for every (sequence, KV head) pair split over several
 * chunks, out = sum_i exp(lse_i - M) o_i / sum_i exp(lse_i - M), M = max lse_i
 * (byteknotlabs "FlashAttention: exact attention without the matrix": partial
 * results rescaled by the running maximum and combined exactly).  Also writes
 * the zero rows (seq_len 0) and NaN rows (invalid length).  Must be given the
 * same seq_lens, shapes and opts as the split call that filled workspace. */
int pkv_lse_combine(const void* workspace, size_t workspace_bytes, const int32_t* seq_lens,
                    int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_blocks_per_seq, void* out, int32_t dtype,
                    const pkv_decode_opts* opts, void* stream);

/* Workspace bytes for the calls above (negative status on bad arguments). */
int64_t pkv_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int32_t n_items);

/* The options the device calls use for these shapes (opts nullable: fields
 * <= 0 take their defaults, given above; the default n_items is also capped
 * at the number of min_chunk_pages chunks in batch * max_blocks_per_seq *
 * n_kv_heads pages), and the workspace they need.  Queries the current HIP
 * device when n_items must be defaulted (needs a GPU). */
int pkv_decode_resolve(int32_t dtype, int32_t head_dim, int32_t n_q_heads, int32_t n_kv_heads,
                       int32_t batch, int32_t max_blocks_per_seq, const pkv_decode_opts* opts,
                       pkv_decode_opts* resolved, int64_t* workspace_bytes);

/* Host mirror of the split plan, for callers that size or inspect partials:
 * seq_lens (host int32 [batch]) -> *chunk_pages (C above), and for every pair
 * (b, h) first_chunk[b * n_kv + h] and last_chunk[b * n_kv + h] (host int32,
 * nullable; -1 for empty sequences).  n_items and min_chunk_pages (>= 1) must
 * already be resolved. */
int pkv_decode_plan(const int32_t* seq_lens, int32_t batch, int32_t n_kv_heads,
                    int32_t block_size, int32_t max_blocks_per_seq, int32_t n_items,
                    int32_t min_chunk_pages, int32_t* chunk_pages, int32_t* first_chunk,
                    int32_t* last_chunk);

/* ------------------------------------------------------------------------ *
 * paged_decode_multi (device): several query tokens per sequence, for
 * verifying a drafted run in one pass (speculative decoding: "Inference
 * Engines" and the CS336 notes run the target once over all drafted tokens)
 * or a chunk of prefill, optionally with a sliding window (CS336 notes,
 * "Local attention & sparse variants": each token attends to the last W).
 * The last q_len cached tokens of sequence b are the queries: query i sits at
 * position seq_lens[b] - q_len + i and attends keys [lo, hi) with
 * hi = seq_lens[b] - q_len + i + 1 and lo = window > 0 ? max(0, hi - window)
 * : 0.  Their K/V must already be appended (pkv_kv_append per token).
 * q, out: [batch][q_len][n_q_heads][head_dim], dtype as pkv_paged_decode_attn.
 * Requires q_len >= 1, window >= 0; a length of 0 gives zero rows, a length
 * below q_len NaN rows.  Pages wholly before every query's window are not
 * read.  Up to 64 query columns per KV head (q_len * n_q_heads / n_kv_heads)
 * the keys are split as in pkv_paged_decode_attn: the workspace and options
 * are its own for n_q_heads * q_len query heads (size it with
 * pkv_decode_resolve / pkv_decode_workspace_bytes given n_q_heads * q_len).
 * Above 64 columns (a prefill chunk, a long drafted run) every 16-column
 * query tile runs over its whole key range in one wavefront, with no
 * partials: workspace, workspace_bytes and opts are then not used (may be
 * NULL / 0), and dtype bf16 and fp32 are both taken.  q_len = 1, window = 0
 * is pkv_paged_decode_attn.
 * ------------------------------------------------------------------------ */
int pkv_paged_decode_multi(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t q_len, int32_t window, float scale, void* out,
                           void* stream, int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                           int32_t dtype, void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts);

/* ------------------------------------------------------------------------ *
 * 8-bit KV cache (device).  Cache quantization changes the bytes per cached
 * element (evaltude docs "Transformer inference mechanics", section "What the
 * KV cache stores per layer"); uniform integer quantization uses a scale and a
 * zero point, with per-group scales (byteknotlabs "Efficient inference",
 * section "Quantization: fewer bytes per weight").  Here each token's K vector
 * and V vector of each KV head is one group, stored as uint8 codes u with
 * x = s * (u - z):
 *   lo = min(min(x), 0), hi = max(max(x), 0), s = (hi - lo) / 255 (1 when
 *   hi == lo), z = rint(-lo / s), u = clamp(rint(x / s) + z, 0, 255),
 * decided in float32 with IEEE division and round-half-to-even.
 * Pools, per page and KV head (caller-owned device memory, 16-byte aligned):
 *   k_codes uint8 [num_pages][n_kv_heads][head_dim / 16][16][16]
 *           (token t, feature 16 c + x at [c][t][x])
 *   v_codes uint8 [num_pages][n_kv_heads][head_dim / 64][4][16][4][4]
 *           (feature d = 64 j + 16 i + n, token t = 4 c + e at [j][c][n][i][e]:
 *           byte 1024 (d / 64) + 256 (t / 4) + 16 (d % 16) + 4 ((d / 16) % 4)
 *           + t % 4 of the tile, so that each lane of a wavefront reads its
 *           operand bytes with 16-byte loads)
 *   meta    float [num_pages][n_kv_heads][4][16]  (k scale, k zero, v scale, v zero per slot)
 * 2 * head_dim + 16 bytes per token and KV head (272 at head_dim 128, against
 * 512 in bf16).  Unused slots may hold anything, NaN scales included.
 *
 * kv_append_q8: quantizes k_new / v_new ([batch][n_kv_heads][head_dim],
 * dtype PKV_BF16 or PKV_F32) into slot positions[b] % 16 of page
 * block_table[b][positions[b] / 16]; invalid positions or page ids skip the
 * sequence, as pkv_kv_append.
 * ------------------------------------------------------------------------ */
int pkv_kv_append_q8(const void* k_new, const void* v_new, void* k_codes, void* v_codes, void* meta,
                     const int32_t* block_table, const int32_t* positions, int32_t batch, int32_t n_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_pages,
                     int32_t dtype, void* stream);

/* Decode over the 8-bit cache: the attention of pkv_paged_decode_attn with
 * K and V the dequantized cache, q and out bf16 [batch][n_q_heads][head_dim].
 * Same semantics, work split, workspace (sized with pkv_decode_resolve and
 * dtype PKV_U8) and options.  The codes enter fp16 matrix products exactly;
 * scores and weights are fp32 with the per-token scales applied to them, so
 * no element is dequantized one by one. */
int pkv_paged_decode_attn_q8(const void* q, const void* k_codes, const void* v_codes, const void* meta,
                             const int32_t* block_table, const int32_t* seq_lens, int32_t n_q_heads,
                             int32_t n_kv_heads, int32_t head_dim, int32_t block_size, float scale, void* out,
                             void* stream, int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                             void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts);

/* The split half alone (partials in the workspace as for pkv_paged_decode_split;
 * merge with pkv_lse_combine, dtype PKV_BF16 or PKV_U8). */
int pkv_paged_decode_split_q8(const void* q, const void* k_codes, const void* v_codes, const void* meta,
                              const int32_t* block_table, const int32_t* seq_lens, int32_t n_q_heads,
                              int32_t n_kv_heads, int32_t head_dim, int32_t block_size, float scale, void* out,
                              void* stream, int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                              void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts);

/* Decode step over the 8-bit cache in one pass: the quantizing append of
 * k_new / v_new (bf16 [batch][n_kv_heads][head_dim], 16-byte aligned) at
 * position seq_lens - 1, done inside the decode kernel, then the decode of
 * pkv_paged_decode_attn_q8.  The wavefront that computes a sequence's last
 * page quantizes the new token exactly as pkv_kv_append_q8 does (same codes,
 * scales and zero points, bit for bit), puts it into its registers and stores
 * it to the pool; so the result and the pool equal pkv_kv_append_q8 at
 * seq_lens - 1 followed by pkv_paged_decode_attn_q8.  One launch (two when
 * the combine kernel is needed, as for the dense step). */
int pkv_decode_step_q8(const void* q, const void* k_new, const void* v_new, void* k_codes, void* v_codes,
                       void* meta, const int32_t* block_table, const int32_t* seq_lens, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, int32_t block_size, float scale, void* out,
                       void* stream, int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                       void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts);

/* ------------------------------------------------------------------------ *
 * copy_blocks (device): copy-on-write of shared blocks (prefix sharing with
 * block-level copy-on-write, CS336 notes "PagedAttention (vLLM)").  For each
 * i < n_pairs, the K and V tiles of every KV head of page src_pages[i] are
 * copied bit for bit to page dst_pages[i] (device int32 arrays), typically
 * the (old, new) pair returned by pkv_seq_reserve_for_write.  Pairs with an
 * id outside [0, num_pages) or src == dst are skipped.  The destination pages
 * must be distinct and must not be source pages of the same call.
 * ------------------------------------------------------------------------ */
int pkv_copy_blocks(void* k_pages, void* v_pages, const int32_t* src_pages,
                    const int32_t* dst_pages, int32_t n_pairs, int32_t n_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t num_pages, int32_t dtype,
                    void* stream);

/* ------------------------------------------------------------------------ *
 * Bandwidth probes (device), for measuring what the HBM path can sustain.
 * pkv_hbm_read_probe streams `bytes` (multiple of 16, buf 16-byte aligned)
 * through 16-byte loads and writes one word per workgroup to sink (device,
 * >= 4 * n_blocks bytes); pkv_copy_probe copies bytes (multiple of 16).
 * ------------------------------------------------------------------------ */
int pkv_hbm_read_probe(const void* buf, size_t bytes, void* sink, int32_t n_blocks, void* stream);
/* The same probe on the 8-bit cache: the chunks, page-id reads and per-tile
 * loads (K codes, V codes and meta, laid out as for pkv_paged_decode_attn_q8)
 * of the 8-bit decode kernel with one query head per KV head, each tile only
 * folded into an XOR written per chunk to sink (device uint32 [n_items],
 * sink_bytes >= 4 * n_items); the ceiling the 8-bit decode is held to.  Page
 * ids outside [0, num_pages) and invalid lengths are skipped. */
int pkv_gather_probe_q8(const void* k_codes, const void* v_codes, const void* meta, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t n_kv_heads, int32_t head_dim, int32_t batch,
                        int32_t max_blocks_per_seq, int32_t num_pages, int32_t n_items, int32_t min_chunk_pages,
                        void* sink, size_t sink_bytes, void* stream);

/* Gather probe: the decode kernel's own tile stream with no arithmetic, for
 * the bandwidth the memory system gives the workload's scattered (page, KV
 * head) tiles ("Transformer inference mechanics", "Knowledge check": measure
 * KV traffic and achieved bandwidth before naming a bottleneck).  It walks
 * the same chunks of the flattened (sequence, KV head, page) order as
 * pkv_paged_decode_attn with one query head per KV head (n_items and
 * min_chunk_pages as in pkv_decode_opts, <= 0 for the defaults), reads every
 * attended page's K and V tiles through the block table with the decode
 * kernel's loads, and writes one XOR of the bytes per chunk to sink (device
 * uint32 [n_items], sink_bytes >= 4 * n_items).  k_pages / v_pages are laid
 * out as for the dense decode, except that the tile of (page p, KV head h)
 * starts p * page_stride_bytes + h * head_stride_bytes after each base
 * (0 and 0: n_kv_heads tiles and one tile, the library's layout; larger
 * multiples of 16 model padded pages, or K and V interleaved per head with
 * v_pages = k_pages + one tile and a head stride of two tiles).  Dense
 * dtypes only; page ids outside [0, num_pages) and invalid lengths are
 * skipped. */
int pkv_gather_probe(const void* k_pages, const void* v_pages, const int32_t* block_table,
                     const int32_t* seq_lens, int32_t n_kv_heads, int32_t head_dim, int32_t batch,
                     int32_t max_blocks_per_seq, int32_t num_pages, int32_t dtype, int64_t page_stride_bytes,
                     int64_t head_stride_bytes, int32_t n_items, int32_t min_chunk_pages, void* sink,
                     size_t sink_bytes, void* stream);
int pkv_copy_probe(void* dst, const void* src, size_t bytes, void* stream);

/* Launch-cost probe: the fixed cost a step pays per kernel, which decides
 * whether a second kernel (the combine of pairs split over more than 96
 * chunks) can be folded into the decode kernel ("Transformer inference
 * mechanics", "Knowledge check": kernel time and launch gaps).  Launches a
 * kernel that does nothing over `grid` workgroups of 256 threads (0: one per
 * compute unit) `iters` times back to back on `stream` after 5 untimed
 * launches, and writes the mean time per launch in microseconds (HIP events)
 * to *us_per_launch (host).  mode 0: ordinary launches; 1: cooperative
 * launches (the whole grid resident at once); 2: cooperative launches whose
 * workgroups meet once at a grid-wide barrier in bar (device int32 [3],
 * zeroed by the caller; on return bar[0] is 0 again, bar[1] counts the
 * barriers passed and bar[2] the polls that gave up, 0 unless the barrier
 * failed).  Blocks until the launches have finished.  Errors: bad mode,
 * grid, iters or pointers; no cooperative launch on the device; a
 * cooperative grid larger than the device holds at once (PKV_ERR_HIP). */
int pkv_launch_probe(int32_t mode, int32_t grid, int32_t iters, int32_t* bar, float* us_per_launch, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
