// Device side of libpkv for gfx950 (CDNA4): kv_append, the split-KV paged
// decode kernel, the log-sum-exp combine and two bandwidth probes, with their
// C-ABI launch entry points.
//
// The operation: for every sequence b and query head hq,
//   out[b][hq] = softmax(scale * q[b][hq] . K^T) V
// over the seq_lens[b] tokens of KV head hq / G held in 16-token pages found
// through the block table (evaltude docs "Transformer inference mechanics",
// "What Q, K, and V do in causal attention" and "MHA versus MQA versus GQA";
// "Inference Engines" chapter 17, "The Breakthrough", for pages and block
// tables).  The softmax is computed online, keeping a running maximum and sum
// so partial results rescale and combine exactly (byteknotlabs "Efficient
// inference", "FlashAttention: exact attention without the matrix"); the KV
// pages are split across wavefronts and merged afterwards (split-KV decode,
// named as FlashDecoding in the CS336 lecture 10 notes).
//
// Mapping onto CDNA4.  One wavefront handles one chunk of pages of one
// (sequence, KV head) pair for 16 query heads of its group at once:
//   * scores S[t][g] = K[t][:] . Q[g][:] for the 16 tokens t of a page is one
//     16x16 MFMA tile (tokens along M, query heads along N, head_dim along K);
//   * the PV product O^T[d][g] += V^T[d][t] P^T[t][g] is D/16 MFMA tiles
//     (head_dim along M, query heads along N, the page's tokens along K).
// Both products put the query head on the MFMA column (lane % 16), so the
// softmax state of head g (running max, sum) lives in the lanes of column g
// and the score tile feeds the PV product as its B operand without any data
// movement.  The page layouts are chosen so that every lane loads its MFMA
// operands straight from HBM with 16-byte (K) or 8/16-byte (V) loads and each
// load instruction of the wavefront covers a contiguous 512 B - 1 KiB:
//   K page [D/X][16][X]: lane l of load i reads bytes 1024 i + 16 l;
//   V page [D][16]:      lane (c = l/16, n = l%16) reads tokens 4c..4c+3 of
//                        feature row 16 nb + n.
// The 8-bit cache stores its V codes in the order the lanes read them
// (q8_v_offset), so they too arrive with 16-byte loads.
// No LDS is needed for the tiles; each K/V tile is read from HBM once and used
// for all query heads of the group from registers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>
#include <type_traits>

#include "pkv_internal.h"

// Device helpers that take register arrays by reference are always inlined:
// a call that the inliner leaves out of line passes the arrays through the
// stack (scratch memory), whose loads wait behind the tile loads in flight.
#define PKV_INLINE __attribute__((always_inline))

// Pages each wavefront keeps in flight ahead of the one it computes.
#ifndef PKV_PREFETCH_PAGES
#define PKV_PREFETCH_PAGES 2
#endif

// Device scratch for callers that cannot allocate (pkv_decode_step_noalloc):
// the decode workspace of those calls, one array per GPU the library runs
// on, held until the process ends.  Host code never uses this name as an
// address: the per-device address comes from hipGetSymbolAddress (see
// scratch_of_current_device).
constexpr size_t kScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309417232121458176568f;
constexpr float kLog2e = 1.442695040888963407359924681001892137f;

// Element i of a 4 x 32-bit register group, reinterpreted as float.  The
// element is copied to a scalar before the reinterpretation: applying
// __builtin_bit_cast to a vector swizzle (v.y) directly compiles to element 0.
template <int I>
__device__ inline float lane_f32(u32x4 v) {
  const uint32_t u = v[I];
  return __builtin_bit_cast(float, u);
}

// ---------------------------------------------------------------------------
// Per-dtype operand handling.
//   NK: 16-byte K (and Q) registers per lane per page; NV: V registers per lane
//   (4 elements each, tokens 4c..4c+3 of one feature row).
// ---------------------------------------------------------------------------
template <bool kBf16, int D>
struct Ops;

// Four floats rounded to bf16 (nearest even) and packed as an MFMA operand.
// Converted two at a time: the compiler turns each two-wide conversion into
// one v_cvt_pk_bf16_f32, but splits a four-wide one into single conversions
// and permutes.  (Ops::pv keeps single conversions: its sum of the rounded
// values reads them one by one, and the split kernel measured 1.6 % slower
// on the 32-layer step with the pairs.)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ inline i16x4 pack_bf16x4(float p0, float p1, float p2, float p3) {
  const bf16x2 lo = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
  const bf16x2 hi = __builtin_convertvector(f32x2{p2, p3}, bf16x2);
  return __builtin_bit_cast(i16x4, u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)});
}

template <int D>
struct Ops<true, D> {  // bfloat16
  static constexpr int ES = 2;
  static constexpr int NK = D * ES / 64;
  static constexpr int NV = D / 16;
  using VReg = u32x2;

  __device__ static f32x4 qk(const u32x4 (&k)[NK], const u32x4 (&q)[NK]) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NK; i += 2) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[i]),
                                                   __builtin_bit_cast(bf16x8, q[i]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[i + 1]),
                                                   __builtin_bit_cast(bf16x8, q[i + 1]), s1, 0, 0, 0);
    }
    return s0 + s1;
  }
  // The same product as one accumulation chain, for callers that compute
  // several independent blocks per page (their chains keep the matrix core
  // busy, and the sum of two chains would cost a register move and an add
  // per score).
  __device__ static f32x4 qk1(const u32x4 (&k)[NK], const u32x4 (&q)[NK]) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NK; ++i)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[i]), __builtin_bit_cast(bf16x8, q[i]),
                                                  s, 0, 0, 0);
    return s;
  }

  // Zero the V elements of tokens >= valid (lane holds tokens 4c..4c+3).
  __device__ static VReg mask_v(VReg v, int c, int valid) {
    uint32_t m0 = (4 * c + 0 < valid ? 0x0000ffffu : 0u) | (4 * c + 1 < valid ? 0xffff0000u : 0u);
    uint32_t m1 = (4 * c + 2 < valid ? 0x0000ffffu : 0u) | (4 * c + 3 < valid ? 0xffff0000u : 0u);
    v.x &= m0;
    v.y &= m1;
    return v;
  }

  // Replaces the element of token 4c + e (e = 0..3) held by this lane.
  __device__ static VReg insert_v(VReg v, int e, uint32_t bits) {
    const uint32_t w = (e & 2) ? v.y : v.x;
    const uint32_t nw = (e & 1) ? ((w & 0x0000ffffu) | (bits << 16)) : ((w & 0xffff0000u) | bits);
    if (e & 2) v.y = nw; else v.x = nw;
    return v;
  }

  // Rounds the four probabilities to the MFMA input type, accumulates the
  // rounded values into l (so the weights that are summed are the weights that
  // are applied) and runs acc[nb] += V^T[nb] * P^T.
  __device__ static void pv(const VReg (&v)[NV], const float (&p)[4], float& l,
                            f32x4 (&acc)[NV]) {
    const bf16x4 pb = {static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1]),
                       static_cast<__bf16>(p[2]), static_cast<__bf16>(p[3])};
    l += (static_cast<float>(pb[0]) + static_cast<float>(pb[1])) +
         (static_cast<float>(pb[2]) + static_cast<float>(pb[3]));
    const i16x4 pk = __builtin_bit_cast(i16x4, pb);
#pragma unroll
    for (int nb = 0; nb < NV; ++nb)
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, v[nb]), pk,
                                                           acc[nb], 0, 0, 0);
  }

  __device__ static void store_out(void* out, size_t elem_off, f32x4 x) {
    const bf16x4 w = {static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1]),
                      static_cast<__bf16>(x[2]), static_cast<__bf16>(x[3])};
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(out) + elem_off) = w;
  }
};

template <int D>
struct Ops<false, D> {  // float32
  static constexpr int ES = 4;
  static constexpr int NK = D * ES / 64;
  static constexpr int NV = D / 16;
  using VReg = u32x4;

  __device__ static f32x4 qk(const u32x4 (&k)[NK], const u32x4 (&q)[NK]) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<0>(k[i]),
                                                lane_f32<0>(q[i]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<1>(k[i]),
                                                lane_f32<1>(q[i]), s1, 0, 0, 0);
      s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<2>(k[i]),
                                                lane_f32<2>(q[i]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<3>(k[i]),
                                                lane_f32<3>(q[i]), s1, 0, 0, 0);
    }
    return s0 + s1;
  }
  __device__ static f32x4 qk1(const u32x4 (&k)[NK], const u32x4 (&q)[NK]) {   // one chain (see Ops<true>)
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      s = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<0>(k[i]), lane_f32<0>(q[i]), s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<1>(k[i]), lane_f32<1>(q[i]), s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<2>(k[i]), lane_f32<2>(q[i]), s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<3>(k[i]), lane_f32<3>(q[i]), s, 0, 0, 0);
    }
    return s;
  }

  __device__ static VReg insert_v(VReg v, int e, uint32_t bits) {
    v.x = e == 0 ? bits : v.x;
    v.y = e == 1 ? bits : v.y;
    v.z = e == 2 ? bits : v.z;
    v.w = e == 3 ? bits : v.w;
    return v;
  }

  __device__ static VReg mask_v(VReg v, int c, int valid) {
    v.x = 4 * c + 0 < valid ? v.x : 0u;
    v.y = 4 * c + 1 < valid ? v.y : 0u;
    v.z = 4 * c + 2 < valid ? v.z : 0u;
    v.w = 4 * c + 3 < valid ? v.w : 0u;
    return v;
  }

  __device__ static void pv(const VReg (&v)[NV], const float (&p)[4], float& l,
                            f32x4 (&acc)[NV]) {
    l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int nb = 0; nb < NV; ++nb) {
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<0>(v[nb]), p[0],
                                                     acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<1>(v[nb]), p[1],
                                                     acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<2>(v[nb]), p[2],
                                                     acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_f32<3>(v[nb]), p[3],
                                                     acc[nb], 0, 0, 0);
    }
  }

  __device__ static void store_out(void* out, size_t elem_off, f32x4 x) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + elem_off) = x;
  }
};

struct DecodeArgs {
  const void* q;
  void* k_pages;           // written only by the fused append
  void* v_pages;
  const void* k_new;       // non-null: fused append of each sequence's last token
  const void* v_new;
  const void* meta;        // 8-bit cache only: per (page, KV head) scales and zero points
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;
  float* part_o;
  float* part_lse;
  int32_t batch, n_q, n_kv, group, max_blocks, num_pages;
  // Query tokens per sequence (the last q_len cached tokens, causal) and the
  // sliding window (0: none); cols = q_len * group columns per KV head, in
  // (query token, query head) order.
  int32_t q_len, window, cols;
  int32_t n_items, min_chunk, waves_per_chunk;
  float scale_log2;
  // Non-null: the chunk that finishes a pair of at most fuse_max_parts
  // chunks last merges its partials (one counter per pair and head block).
  // Points at the workspace's last int32 word; the counters lie below it
  // (see merge_counter).
  int32_t* counters;
  int32_t fuse_max_parts;
  // Per-sequence page prefix [batch + 1] in the workspace: written by the
  // split kernel's first workgroup, read by the combine kernel.
  int32_t* prefix;
  // Dynamic schedule: the counter chunks are taken from (zero between launches).
  int32_t* work;
  // Static schedule with the in-kernel merge: pairs whose chunks all belong to
  // one workgroup are merged through LDS (wg_lds_offset: int32 offset of the
  // partial slots in the kernel's dynamic LDS).
  int32_t wg_merge, wg_lds_offset;
  // Split kernel's per-wavefront LDS after the prefix (int32 words):
  // held_cap slots of held_tok_words (fused append's tokens; 0 without
  // append), then held_cap result slots of held_res_words (0: results are
  // written at once); held_wave_words per wavefront in all.
  int32_t held_cap, held_tok_words, held_res_words, held_wave_words;
};

// Pages per sequence (those from its first attended block, see
// pages_of_range), exclusive prefix over the batch, into LDS (whole
// workgroup).  s_prefix[b] = pages of sequences before b; s_prefix[batch] =
// total.  A length outside [q_len, 16 * max_blocks] counts as zero pages.
__device__ void build_prefix(const int32_t* __restrict__ seq_lens, int batch, int max_blocks, int q_len,
                             int window, int32_t* s_prefix, int32_t* s_wsum) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int per = (batch + nthr - 1) / nthr;
  const int b0 = min(batch, tid * per);
  const int b1 = min(batch, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += pages_of_range(seq_lens[b], max_blocks, q_len, window);
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  int x = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) s_wsum[wid] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += s_wsum[w];
  int run = base + x - local;
  for (int b = b0; b < b1; ++b) {
    s_prefix[b] = run;
    run += pages_of_range(seq_lens[b], max_blocks, q_len, window);
  }
  if (tid == nthr - 1) s_prefix[batch] = base + x;
  __syncthreads();
}

// Largest b in [0, batch) with n_kv * prefix[b] <= f (f < total): the sequence
// that owns flattened page f; it always holds at least one page.
__device__ inline int find_seq(const int32_t* s_prefix, int batch, int n_kv, int f) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (n_kv * s_prefix[mid] <= f) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Wave-uniform value in a scalar register (every lane holds the same value).
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// The block table is read-only during a launch; reading it through the
// constant address space with a wave-uniform index makes every page-id read a
// scalar load (scalar cache, its own counter), so it never waits behind the
// vector loads of K/V tiles in flight.
typedef __attribute__((address_space(4))) const int32_t const_i32;

// Length of sequence b (b wave-uniform), read the same way: a vector load
// here would be waited for together with every tile load issued before it.
__device__ inline int seq_len_of(const DecodeArgs& a, int b) {
  return ((const const_i32*)a.seq_lens)[b];
}

template <bool kBf16, int D>
struct PageRegs {
  using O = Ops<kBf16, D>;
  u32x4 k[O::NK];
  typename O::VReg v[O::NV];
};

// Buffer-resource word 3 for raw (untyped) buffer loads on CDNA: 32-bit data
// format, no swizzle, no index stride.
#ifndef PKV_RSRC_WORD3
#define PKV_RSRC_WORD3 0x00020000
#endif
// Cache-policy bits for device scope (SC1 set, SC0 clear): the access is
// coherent across the XCDs, whose L2 caches are not coherent with each
// other.  Used for the split partials that another workgroup merges in the
// same launch.
constexpr int kDeviceScope = 16;
// s_waitcnt immediate (gfx9 layout) waiting for vmcnt = 0 only (expcnt and
// lgkmcnt fields at their maxima): all of this wavefront's vector memory
// operations, stores included, have completed.
constexpr int kWaitVmcnt0 = 0x0F70;

// Cache-policy bits of the K/V tile loads: non-temporal (each tile is read
// once per launch, so it should not displace other lines; ~10% faster than
// the default policy on the 16 x 4096 MHA layer).
#ifndef PKV_KV_LOAD_AUX
#define PKV_KV_LOAD_AUX 2
#endif
// Cache policy when several wavefronts (one per 16-head block of a large
// group) read the same tiles at about the same time: default, so that the
// first reader's lines serve the others from the caches.
#ifndef PKV_KV_LOAD_AUX_GROUPED
#define PKV_KV_LOAD_AUX_GROUPED 0
#endif

// Issues the loads of one (page, KV head) tile.  kbase/vbase are wave-uniform
// and become the base of a buffer resource whose range is exactly one tile, so
// the per-lane offsets (koff = 16 * lane, voff = elem * (16 n + 4 c)) stay in
// one register and an offset past the tile reads zero instead of faulting.
// range = 0 issues the same loads without touching memory (they return
// zeros): used past the end of a range and for page ids outside the pool.
template <bool kBf16, int D, int kAux = PKV_KV_LOAD_AUX>
__device__ inline void load_page(PageRegs<kBf16, D>& r, const char* kbase, const char* vbase,
                                 uint32_t koff, uint32_t voff, int range) {
  using O = Ops<kBf16, D>;
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase), 0, range, PKV_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase), 0, range, PKV_RSRC_WORD3);
#pragma unroll
  for (int i = 0; i < O::NK; ++i)
    r.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, koff + 1024 * i, 0, kAux);
#pragma unroll
  for (int nb = 0; nb < O::NV; ++nb) {
    if constexpr (kBf16)
      r.v[nb] = __builtin_amdgcn_raw_buffer_load_b64(vr, voff + O::ES * 16 * kBlock * nb, 0, kAux);
    else
      r.v[nb] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff + O::ES * 16 * kBlock * nb, 0, kAux);
  }
}

// Largest growth of a score (log2 units) over the running maximum that is
// accepted without rescaling: exponentials stay <= 2^8, far from overflow in
// fp32 accumulation and exactly representable in range for bf16.
constexpr float kLazyRescale = 8.0f;
// Running maximum of a column before it has seen any key.  Finite, so that a
// column whose keys are all masked so far (a later query token whose window
// starts past the page, or a chunk wholly past a query token's position)
// weighs its scores exp2(-inf - kNoKeysMax) = 0 and rescales by exp2(0) = 1,
// where -inf would give exp2(-inf - -inf) = NaN.  Scores are far above it.
constexpr float kNoKeysMax = -1.0e30f;

// One page of the online softmax for the 16 query heads of this wavefront.
// The running maximum m of a query head is shared by the four lanes of its
// column; it is raised (and the sum and accumulator rescaled) only when some
// score of the page exceeds it by more than kLazyRescale, which one wave-wide
// vote detects.  Between raises, m is an upper bound minus at most 8, so
// exp2(x - m) <= 2^8, and the final division by the sum is unchanged.
//
// Masks: when `cut` (scalar: some column's key range [lo, hi) ends or starts
// inside this page), the lane keeps token tok0 + 4c + i only inside its own
// column's range; V elements of slots past the sequence (valid < 16, last
// page only) are zeroed, since 0 * NaN would poison the sums.
template <bool kBf16, int D, bool kMulti>
__device__ inline void compute_page(PageRegs<kBf16, D>& r, int valid, bool cut, int tok0, int hi, int lo,
                                    const u32x4 (&qreg)[Ops<kBf16, D>::NK], float scale_log2,
                                    int c, float& m, float& l,
                                    f32x4 (&acc)[Ops<kBf16, D>::NV]) {
  using O = Ops<kBf16, D>;
  f32x4 s = O::qk(r.k, qreg);   // lane (c, n): tokens 4c + i, column n
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = s[i] * scale_log2;
  if (cut) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tok0 + 4 * c + i;
      const bool in = kMulti ? (t < hi && t >= lo) : 4 * c + i < valid;
      x[i] = in ? x[i] : -INFINITY;
    }
  }
  if (valid < kBlock) {
#pragma unroll
    for (int nb = 0; nb < O::NV; ++nb) r.v[nb] = O::mask_v(r.v[nb], c, valid);
  }
  const float pm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (__builtin_amdgcn_ballot_w64(pm > m + kLazyRescale) != 0) {
    float cm = fmaxf(pm, __shfl_xor(pm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));
    const float mn = fmaxf(m, cm);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int nb = 0; nb < O::NV; ++nb) acc[nb] *= alpha;
    m = mn;
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m);
  O::pv(r.v, p, l, acc);
}

// The decode kernels' dynamic LDS, seen as floats (the workgroup-merge slots).
extern __shared__ float lds_f32[];

// Pairs whose partial this wavefront wrote and that it may have to merge:
// only a chunk's first and last segments can belong to pairs that span
// several chunks, so at most two.  Merged after the page loop, which keeps
// the merge's registers out of it.
struct PendingMerges {
  int n = 0;
  int b0 = 0, h0 = 0, first0 = 0, nparts0 = 0;
  int b1 = 0, h1 = 0, first1 = 0, nparts1 = 0;
  // Selects, not a branch on n: a branch made the compiler keep the two
  // entries as an array indexed at run time, in scratch memory, whose stores
  // then queued behind the tile loads.
  __device__ void add(int b, int h, int first, int nparts) {
    const bool f = n == 0;
    b0 = f ? b : b0; h0 = f ? h : h0; first0 = f ? first : first0; nparts0 = f ? nparts : nparts0;
    b1 = f ? b1 : b; h1 = f ? h1 : h; first1 = f ? first1 : first; nparts1 = f ? nparts1 : nparts;
    n = n < 2 ? n + 1 : 2;
  }
  // Pairs whose chunks all run in this workgroup (static schedule): their
  // partials go to LDS slots, and the wavefront holding a pair's first chunk
  // merges it after a workgroup barrier.  wg_base: float index in the
  // dynamic LDS of this workgroup's slots (slot 2 w + k: wavefront w's first
  // (k = 0) or last (k = 1) segment), partial rows float [8][cols][D] then
  // lse float [8][cols]; -1 when off.  An index, not a pointer: a pointer
  // kept across the page loop lives in a vector register.
  int wg_base = -1;
  int wg_first = -1;            // chunk of the workgroup's first wavefront
  int nw = 0, wb = 0, wh = 0, wfirst = 0, wparts = 0;   // the pair this wavefront merges
  __device__ bool in_workgroup(int first_chunk, int last_chunk) const {
    return wg_base >= 0 && first_chunk >= wg_first && last_chunk < wg_first + kWavesPerGroup;
  }
};

// The same for the dynamic schedule, where a wavefront takes any number of
// chunks: the pairs are listed in this wavefront's slice of LDS (b, h, first
// chunk, parts) until they are counted, at the end of its work or when the
// list is full.
struct PendingList {
  int4* list;   // kMaxPending entries
  int n = 0;
  int wg_base = -1, wg_first = -1, nw = 0, wb = 0, wh = 0, wfirst = 0, wparts = 0;
  __device__ bool in_workgroup(int, int) const { return false; }   // chunks move between workgroups
  __device__ void add(int b, int h, int first, int nparts) {
    if ((threadIdx.x & (kWave - 1)) == 0) list[n] = make_int4(b, h, first, nparts);
    ++n;
  }
};

// Output row of column g = (query token qi, query head gq) of KV head h of
// sequence b, in out [batch][q_len][n_q][D].
// One query token (kMulti false): column g is query head g of the group.
template <bool kMulti>
__device__ inline size_t out_row(const DecodeArgs& a, int b, int h, int g) {
  if constexpr (!kMulti) return static_cast<size_t>(b) * a.n_q + h * a.group + g;
  const int qi = g / a.group;
  const int gq = g - qi * a.group;
  return (static_cast<size_t>(b) * a.q_len + qi) * a.n_q + h * a.group + gq;
}

// Writes one segment's normalised result o (lane (c, n): features
// 16 nb + 4c .. +3 of head gb*16 + n) and its natural-log lse: the output rows
// when the pair lies in a single chunk, otherwise this chunk's partial, which
// the last of the pair's chunks to finish then merges (if counters are on).
template <bool kOutBf16, int D, bool kMulti, class Pending>
PKV_INLINE __device__ void emit_segment(const DecodeArgs& a, int b, int h, int gb, int n_pages, int seg_start, int chunk,
                             int C, const f32x4 (&o)[D / 16], float lse, int lane, Pending& pending) {
  using O = Ops<kOutBf16, D>;
  const int c = lane >> 4;
  const uint32_t n = lane & 15;
  const int g = gb * 16 + static_cast<int>(n);      // column (query token, query head)
  const int first_chunk = seg_start / C;
  const int last_chunk = (seg_start + n_pages - 1) / C;
  if (first_chunk == last_chunk) {
    if (g >= a.cols) return;
    const size_t row = out_row<kMulti>(a, b, h, g) * D;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) O::store_out(a.out, row + 16 * nb + 4 * c, o[nb]);
    return;
  }
  if (pending.in_workgroup(first_chunk, last_chunk)) {
    // Slot 0 if the pair began before this chunk (the chunk's first
    // segment), else 1; lanes of columns past the group store nothing.
    const int which = seg_start < chunk * C ? 0 : 1;
    const int cols = a.cols;
    const int slot = (chunk - pending.wg_first) * 2 + which;
    const int base = uni(pending.wg_base);
    if (static_cast<int>(n) < cols) {
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb)
        *reinterpret_cast<f32x4*>(lds_f32 + base + (slot * cols + n) * lds_row(D) + 16 * nb + 4 * c) = o[nb];
      if (c == 0) lds_f32[base + 2 * kWavesPerGroup * cols * lds_row(D) + slot * cols + n] = lse;
    }
    if (which == 1) {
      pending.nw = 1;
      pending.wb = b;
      pending.wh = h;
      pending.wfirst = first_chunk;
      pending.wparts = last_chunk - first_chunk + 1;
    }
    return;
  }
  // Device-scope stores: written through to the point where every XCD sees
  // them, so the chunk that merges (possibly on another XCD) reads them
  // without any cache-wide write-back or invalidation.  The row resource's
  // range ends at the group's last head, which masks the lanes of heads past it.
  const size_t slot = static_cast<size_t>(chunk) + static_cast<size_t>(b) * a.n_kv + h;
  const int rows = min(16, a.cols - gb * 16);
  const size_t row0 = slot * a.cols + gb * 16;
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(a.part_o + row0 * D, 0, rows * D * 4, PKV_RSRC_WORD3);
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[nb]), ro, 4 * (n * D + 16 * nb + 4 * c), 0,
                                           kDeviceScope);
  if (c == 0) {
    const __amdgpu_buffer_rsrc_t rl =
        __builtin_amdgcn_make_buffer_rsrc(a.part_lse + row0, 0, rows * 4, PKV_RSRC_WORD3);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), rl, 4 * n, 0, kDeviceScope);
  }
  const int nparts = last_chunk - first_chunk + 1;
  if (a.counters != nullptr && nparts <= a.fuse_max_parts) pending.add(b, h, first_chunk, nparts);
}

// Results of segments that end inside the page loop (pairs that end in the
// middle of the chunk), held in this wavefront's LDS until its tile stream
// has drained, for the same reason as the new tokens below: a result
// written at once holds back the waits for every later tile.  Slot i at
// float index base + i * words: o rows [cols][D], lse [cols], then
// (b, h, n_pages, seg_start) in the last four words; up to cap slots, a
// result past them is written at once.  Indices, not pointers (see
// PendingMerges::wg_base).
struct HeldResults {
  int n = 0, cap = 0, base = 0, words = 0;
  // Rows 16 blk .. 16 blk + 15 of slot n (head block blk of the wavefront's
  // one or two): the block's normalised result o and its lse.
  template <int D>
  PKV_INLINE __device__ void put_block(const DecodeArgs& a, int blk, const f32x4 (&o)[D / 16], float lse, int lane) {
    const int c = lane >> 4, row = 16 * blk + (lane & 15);
    const int cols = a.cols;
    const int sb = uni(base + n * words);
    if (row < cols) {
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb)
        *reinterpret_cast<f32x4*>(lds_f32 + sb + row * lds_row(D) + 16 * nb + 4 * c) = o[nb];
      if (c == 0) lds_f32[sb + cols * lds_row(D) + row] = lse;
    }
  }
  // Closes slot n with the segment's coordinates.
  PKV_INLINE __device__ void commit(int b, int h, int n_pages, int seg_start, int lane) {
    const int sb = uni(base + n * words);
    if (lane == 0) *reinterpret_cast<int4*>(lds_f32 + sb + words - 4) = make_int4(b, h, n_pages, seg_start);
    ++n;
  }
  // Writes the held results (see emit_segment), in the order they ended:
  // block blk of each as head block gb + blk; the pairs to merge are listed
  // in `pending` by block 0 (the other block's pairs are the same).
  template <bool kOutBf16, int D, bool kMulti, int kNB, class Pending>
  PKV_INLINE __device__ void emit_all(const DecodeArgs& a, int gb, int chunk, int C, int lane, Pending& pending,
                                      Pending& unused) {
    const int c = lane >> 4, col = lane & 15;
    for (int i = 0; i < n; ++i) {
      const int sb = uni(base + i * words);
      const int4 d = *reinterpret_cast<const int4*>(lds_f32 + sb + words - 4);
#pragma unroll
      for (int blk = 0; blk < kNB; ++blk) {
        if (blk > 0 && (gb + blk) * 16 >= a.cols) continue;
        const int rc = min(16 * blk + col, a.cols - 1);   // lanes past the group read a valid row and write nothing
        f32x4 o[D / 16];
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb)
          o[nb] = *reinterpret_cast<const f32x4*>(lds_f32 + sb + rc * lds_row(D) + 16 * nb + 4 * c);
        const float lse = lds_f32[sb + a.cols * lds_row(D) + rc];
        emit_segment<kOutBf16, D, kMulti>(a, uni(d.x), uni(d.y), gb + blk, uni(d.z), uni(d.w), chunk, C, o, lse,
                                          lane, blk == 0 ? pending : unused);
      }
    }
    n = 0;
  }
};

// New tokens of a fused append, held until the wavefront has no tile loads
// in flight.  Vector memory operations retire in order, so a store issued in
// the middle of the tile stream holds back the waits for every later tile;
// measured on MI355X the token's stores cost 8 us of the 181-us GQA layer
// when issued at the pair's last page (writing the whole 8-KiB tile back
// instead, in full lines, cost as much).  A token waits in a slot of this
// wavefront's LDS (K row, then V row as 32-bit words, then its destination),
// which costs no registers; LDS accesses have their own counter.  A token
// handed to an occupied slot first pushes the slot's token out to the pool.
// kDefer false (kernels whose sibling wavefronts share a chunk): the token is
// stored as soon as it is handed over.
template <bool kBf16, int D, bool kDefer = true>
struct HeldToken {
  using O = Ops<kBf16, D>;
  static constexpr int kRowWords = D * O::ES / 4 + D;   // K row, then D words of V
  static constexpr int kSlotWords = kRowWords + 8;      // + K and V tile addresses, slot of the token
  static_assert(kSlotWords <= kHeldWords, "a held token fits its LDS slot");
  uint32_t* lds;        // slot 0 of this wavefront; slot i at lds + i * kSlotWords
  uint32_t mask = 0;    // slots holding a token (uniform)

  // K: the 16-byte pieces of slot s_new (lanes with lane % 16 == s_new, as
  // loaded); V: its element of every feature row (lanes with lane / 16 ==
  // s_new / 4).
  __device__ static void store_regs(const u32x4 (&k)[O::NK], const uint32_t (&v)[O::NV], char* kbase, char* vbase,
                                    int s_new, int lane) {
    const int c = lane >> 4, n = lane & 15;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc(kbase, 0, kBlock * D * O::ES, PKV_RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(vbase, 0, kBlock * D * O::ES, PKV_RSRC_WORD3);
    if (n == s_new) {
#pragma unroll
      for (int i = 0; i < O::NK; ++i) __builtin_amdgcn_raw_buffer_store_b128(k[i], kr, 16u * lane + 1024 * i, 0, 0);
    }
    if (c == (s_new >> 2)) {
      const uint32_t vo = O::ES * (n * kBlock + s_new);
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) {
        if constexpr (kBf16)
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v[nb]), vr, vo + O::ES * 16 * kBlock * nb, 0,
                                                0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(v[nb], vr, vo + O::ES * 16 * kBlock * nb, 0, 0);
      }
    }
  }

  // Writes the token of slot i to the pool and frees the slot.
  __device__ void store_slot(int i, int lane) {
    mask &= ~(1u << i);
    const int c = lane >> 4, n = lane & 15;
    const uint32_t* w = lds + i * kSlotWords;
    const u32x4* lk = reinterpret_cast<const u32x4*>(w);
    u32x4 k[O::NK];
    uint32_t v[O::NV];
#pragma unroll
    for (int j = 0; j < O::NK; ++j) k[j] = lk[4 * j + c];
#pragma unroll
    for (int nb = 0; nb < O::NV; ++nb) v[nb] = w[D * O::ES / 4 + 16 * nb + n];
    const u32x4 dst = *reinterpret_cast<const u32x4*>(w + kRowWords);
    auto u = [](uint32_t x) { return static_cast<uint64_t>(static_cast<uint32_t>(uni(static_cast<int>(x)))); };
    const uint64_t kb = (u(dst.y) << 32) | u(dst.x);
    const uint64_t vb = (u(dst.w) << 32) | u(dst.z);
    const int s_new = uni(static_cast<int>(w[kRowWords + 4]));
    store_regs(k, v, reinterpret_cast<char*>(kb), reinterpret_cast<char*>(vb), s_new, lane);
  }

  // Takes the token bound for slot s_new of the tiles at kbase / vbase: k[i]
  // in lanes (c, any n) is K piece 4i + c; v[nb] in lanes (any c, n) is V
  // element 16 nb + n.  It is held in LDS slot `slot`, or stored at once if
  // `now` (the caller has no more tiles to stream, or no slot).
  __device__ void take(const u32x4 (&k)[O::NK], const uint32_t (&v)[O::NV], char* kbase, char* vbase, int s_new,
                       int slot, int lane, bool now) {
    if (!kDefer || now) {
      store_regs(k, v, kbase, vbase, s_new, lane);
      return;
    }
    if ((mask >> slot) & 1u) store_slot(slot, lane);
    mask |= 1u << slot;
    const int c = lane >> 4, n = lane & 15;
    uint32_t* w = lds + slot * kSlotWords;
    u32x4* lk = reinterpret_cast<u32x4*>(w);
    if (n == 0) {
#pragma unroll
      for (int i = 0; i < O::NK; ++i) lk[4 * i + c] = k[i];
    }
    if (c == 0) {
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) w[D * O::ES / 4 + 16 * nb + n] = v[nb];
    }
    if (lane == 0) {
      const uint64_t kb = reinterpret_cast<uint64_t>(kbase), vb = reinterpret_cast<uint64_t>(vbase);
      *reinterpret_cast<u32x4*>(w + kRowWords) = u32x4{static_cast<uint32_t>(kb), static_cast<uint32_t>(kb >> 32),
                                                        static_cast<uint32_t>(vb), static_cast<uint32_t>(vb >> 32)};
      w[kRowWords + 4] = static_cast<uint32_t>(s_new);
    }
  }

  // Writes every held token to the pool, in slot order.
  __device__ void store(int lane) {
    if constexpr (kDefer) {
      while (mask != 0) store_slot(__builtin_ctz(mask), lane);
    }
  }
};

// One segment: the pages of one (sequence b, KV head h) pair that one chunk
// covers, for the 16 query heads gblk*16 .. gblk*16+15 (lane column n = head
// gblk*16 + n).  Holds the query operand, the online-softmax state and, when
// the segment ends with the pair's last page and the step appends, the new
// token's K/V in the lanes that hold its slot.
template <bool kBf16, int D, bool kMulti>
struct Segment {
  using O = Ops<kBf16, D>;
  static constexpr int kTileBytes = kBlock * D * O::ES;
  int b, h, gb, g, hq, len, n_pages, s_new, fb, q_len, window, hi, lo;
  bool g_ok, append;
  u32x4 qreg[O::NK];
  u32x4 knew[O::NK];
  uint32_t vnew[O::NV];
  float m, l;
  f32x4 acc[O::NV];

  __device__ void begin(const DecodeArgs& a, int b_, int h_, int n_pages_, int fb_, bool ends_pair, int gblk,
                        int lane) {
    const int c = lane >> 4, n = lane & 15;
    b = b_;
    h = h_;
    n_pages = n_pages_;
    fb = fb_;
    gb = gblk;
    // Column g = (query token qi, query head gq) of this KV head.
    g = gblk * 16 + n;
    g_ok = g < a.cols;
    const int qi = kMulti ? g / a.group : 0;
    const int gq = g - qi * a.group;
    hq = h * a.group + gq;
    len = seq_len_of(a, b);
    q_len = kMulti ? a.q_len : 1;
    window = kMulti ? a.window : 0;
    hi = len - q_len + qi + 1;
    lo = window > 0 ? max(0, hi - window) : 0;
    // Query operand: lane (c, n) holds q[b][qi][hq][(4i + c) * X .. +X) for each i
    // (columns past the group read row 0 and hold zeros).
    const size_t qrow = g_ok ? (static_cast<size_t>(b) * q_len + qi) * a.n_q + hq : 0;
    const char* qb = static_cast<const char*>(a.q) + qrow * D * O::ES;
#pragma unroll
    for (int i = 0; i < O::NK; ++i) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(qb + 16 * (4 * i + c));
      qreg[i] = g_ok ? t : u32x4{0u, 0u, 0u, 0u};
    }
    m = kNoKeysMax;
    l = 0.f;
#pragma unroll
    for (int nb = 0; nb < O::NV; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Fused append: the segment holding the pair's last page also holds the
    // new token (slot (len - 1) % 16 of that page).
    append = a.k_new != nullptr && ends_pair;
    s_new = (len - 1) & (kBlock - 1);
    if (append) {
      const size_t row = (static_cast<size_t>(b) * a.n_kv + h) * D;
      const char* kn = static_cast<const char*>(a.k_new) + row * O::ES;
#pragma unroll
      for (int i = 0; i < O::NK; ++i) knew[i] = *reinterpret_cast<const u32x4*>(kn + 16 * (4 * i + c));
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) {
        if constexpr (kBf16)
          vnew[nb] = static_cast<const uint16_t*>(a.v_new)[row + 16 * nb + n];
        else
          vnew[nb] = static_cast<const uint32_t*>(a.v_new)[row + 16 * nb + n];
      }
    }
  }

  // Puts the new token into the tile registers of the pair's last page: the
  // lanes whose K pieces belong to slot s_new (lane % 16 == s_new) and whose V
  // elements are tokens 4c..4c+3 with c = s_new / 4.
  __device__ void patch(PageRegs<kBf16, D>& r, int lane) const {
    const int c = lane >> 4, n = lane & 15;
    if (n == s_new) {
#pragma unroll
      for (int i = 0; i < O::NK; ++i) r.k[i] = knew[i];
    }
    if (c == (s_new >> 2)) {
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) r.v[nb] = O::insert_v(r.v[nb], s_new & 3, vnew[nb]);
    }
  }

  // The fused append on the pair's last page: the new token into the page
  // registers, and, if `store`, handed to `held` for page pg.
  template <class Held>
  __device__ void append_token(PageRegs<kBf16, D>& r, Held& t, char* kpool, char* vpool, size_t page_stride, int pg,
                               bool store, int slot, int lane, bool now) const {
    patch(r, lane);
    if (store) hold(t, kpool, vpool, page_stride, pg, slot, lane, now);
  }

  // Hands the new token (already in knew/vnew) to `held` (slot `slot`), to
  // be written to page pg of the pool (kpool/vpool point at head h of page 0)
  // once the wavefront's tile stream has drained, or at once if `now`.
  template <bool kDefer>
  __device__ void hold(HeldToken<kBf16, D, kDefer>& t, char* kpool, char* vpool, size_t page_stride, int pg,
                       int slot, int lane, bool now) const {
    const size_t off = static_cast<size_t>(pg) * page_stride;
    t.take(knew, vnew, kpool + off, vpool + off, s_new, slot, lane, now);
  }

  // Page j of the segment holds sequence tokens 16 (fb + j) .. +15.  Columns
  // see keys [lo, hi): the smallest hi is len - q_len + 1, the largest lo is
  // len - window.  One query token (kMulti false): every column sees [0, len)
  // and only the last page is cut.
  __device__ void page(PageRegs<kBf16, D>& r, int j, float scale_log2, int lane) {
    if constexpr (kMulti) {
      const int tok0 = kBlock * (fb + j);
      const bool cut = tok0 + kBlock > len - q_len + 1 || (window > 0 && tok0 < len - window);
      compute_page<kBf16, D, true>(r, len - tok0, cut, tok0, hi, lo, qreg, scale_log2, lane >> 4, m, l, acc);
    } else {
      const int valid = len - kBlock * j;
      compute_page<kBf16, D, false>(r, valid, valid < kBlock, 0, 0, 0, qreg, scale_log2, lane >> 4, m, l, acc);
    }
  }

  // Normalises the segment's result in place and writes it (see
  // emit_segment); the segment is closed afterwards.
  // Normalises the result in place and returns its natural-log lse.
  PKV_INLINE __device__ float normalise(bool bad) {
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = bad ? NAN : (!kMulti || lt > 0.f ? 1.0f / lt : 0.f);   // no key seen: zero row, lse -inf
#pragma unroll
    for (int nb = 0; nb < O::NV; ++nb) acc[nb] *= inv;
    return bad ? NAN : (m + __log2f(lt)) * kLn2;
  }
  template <class Pending>
  PKV_INLINE __device__ void finish(const DecodeArgs& a, int seg_start, int chunk, int C, bool bad, int lane,
                         Pending& pending) {
    const float lse = normalise(bad);
    emit_segment<kBf16, D, kMulti>(a, b, h, gb, n_pages, seg_start, chunk, C, acc, lse, lane, pending);
  }
};

// Arrival of this wavefront's partials for (b, h, head block gb).  The
// partials were written with device-scope stores; once they have completed
// (vmcnt 0: every vector memory operation of this wavefront done), one lane
// counts the arrival with a device-scope atomic.
//
// Why this orders the merge on gfx950 without agent-scope fences: a fence
// with release semantics at agent scope is, on this architecture, an L2
// write-back of lines written with the default policy followed by a wait
// for vmcnt 0, and an acquire fence is an invalidation of the caches
// between the wave and memory.  Every access of this protocol carries the
// agent-scope policy bits itself instead: the partial stores are written
// through the writer's L2 (and are counted complete by vmcnt only once the
// device-coherent level has them), the counter atomic is performed at that
// level, and the merge's loads do not hit a stale line in the reader's L1
// or L2.  The wait for vmcnt 0 before the atomic is the release's wait; the
// control dependence of the loads on the atomic's result, plus the
// compiler barriers around both, keeps every load after it.  The
// write-back and invalidation are then redundant; as fences they cover
// whole caches and cost 30 % on the 16 x 4096 MHA layer.  The wavefront that brings
// the count to nparts reads the nparts partials with device-scope loads,
// merges them in chunk order (out = sum_i w_i o_i / sum_i w_i, w_i =
// exp(lse_i - max lse), the combine kernel's formula) and resets the counter
// for the next call.  No wavefront waits for another.
__device__ inline int32_t* merge_counter(const DecodeArgs& a, int b, int h, int gb) {
  return a.counters - 1 - ((static_cast<ptrdiff_t>(b) * a.n_kv + h) * kMaxWavesPerChunk + gb);
}

// Counts this wavefront's arrivals for its (at most two) pending pairs, both
// atomics in flight together, after all its stores have completed; returns
// a bit per pending pair for which it arrived last.
__device__ inline int arrive(const DecodeArgs& a, const PendingMerges& pm, int gb, int lane) {
  // Compiler-level barrier: the partial stores stay before the wait, and
  // (below) the merge's loads after the atomic's result.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  int o0 = 0, o1 = 0;
  if (lane == 0) {
    if (pm.n > 0)
      o0 = __hip_atomic_fetch_add(merge_counter(a, pm.b0, pm.h0, gb), 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    if (pm.n > 1)
      o1 = __hip_atomic_fetch_add(merge_counter(a, pm.b1, pm.h1, gb), 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  }
  o0 = __shfl(o0, 0);
  o1 = __shfl(o1, 0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return (pm.n > 0 && o0 == pm.nparts0 - 1 ? 1 : 0) | (pm.n > 1 && o1 == pm.nparts1 - 1 ? 2 : 0);
}

// Merges nparts partials of one (sequence b, KV head h, head block gb) and
// writes the output rows: out = sum_i w_i o_i / sum_i w_i, w_i = exp(lse_i -
// max lse).  One pass, kMergeGroup parts per round trip: all their loads are
// issued before any is used, and the running maximum rescales the sums (the
// same identity as the page loop).  load(i, l, v) fetches part i's lse and
// this lane's features (lane (c, n): features 16 nb + 4c .. +3 of column
// gb * 16 + n); parts past nparts read zeros and weigh nothing.  The same
// arithmetic serves partials in global memory and in LDS, so both give the
// same bits.  32 f32x4 registers of loads per group by default; fewer where
// the caller holds other live registers.
template <bool kBf16, int D, bool kMulti, int kGroupParts, class Load>
PKV_INLINE __device__ void merge_core(const DecodeArgs& a, int b, int h, int gb, int nparts, int lane, Load load) {
  using O = Ops<kBf16, D>;
  const uint32_t c = lane >> 4, n = lane & 15;
  const int g = gb * 16 + static_cast<int>(n);   // column
  const bool g_ok = g < a.cols;
  constexpr int kMergeGroup = kGroupParts > 0 ? kGroupParts : 32 / O::NV;
  float mx = kNoKeysMax, den = 0.f;   // parts that saw no key have lse -inf and weigh 0
  f32x4 o[O::NV];
#pragma unroll
  for (int nb = 0; nb < O::NV; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < nparts; i0 += kMergeGroup) {
    float l[kMergeGroup];
    f32x4 v[kMergeGroup][O::NV];
#pragma unroll
    for (int u = 0; u < kMergeGroup; ++u) load(i0 + u, l[u], v[u]);
    float gm = mx;
#pragma unroll
    for (int u = 0; u < kMergeGroup; ++u) gm = i0 + u < nparts ? fmaxf(gm, l[u]) : gm;
    const float alpha = __expf(mx - gm);   // 0 on the first group (mx = -inf)
    den *= alpha;
#pragma unroll
    for (int nb = 0; nb < O::NV; ++nb) o[nb] *= alpha;
#pragma unroll
    for (int u = 0; u < kMergeGroup; ++u) {
      const float w = i0 + u < nparts ? __expf(l[u] - gm) : 0.f;
      den += w;
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) o[nb] += w * v[u][nb];
    }
    mx = gm;
  }
  if (g_ok) {
    const float inv = 1.0f / den;
    const size_t row = out_row<kMulti>(a, b, h, g) * D;
#pragma unroll
    for (int nb = 0; nb < O::NV; ++nb) O::store_out(a.out, row + 16 * nb + 4 * c, o[nb] * inv);
  }
}

// The global merge: the partials of chunks first_chunk .. + nparts - 1, read
// with device-scope loads (their writers may be on other XCDs); then the
// pair's arrival counter is reset for the next call.
template <bool kBf16, int D, bool kMulti, int kGroupParts = 0>
__device__ void merge_pair(const DecodeArgs& a, int b, int h, int gb, int first_chunk, int nparts, int lane) {
  using O = Ops<kBf16, D>;
  int32_t* ctr = merge_counter(a, b, h, gb);
  const uint32_t c = lane >> 4, n = lane & 15;
  const uint32_t G = a.cols;                      // partial rows per slot
  const size_t row0 = (static_cast<size_t>(first_chunk) + static_cast<size_t>(b) * a.n_kv + h) * G + gb * 16;
  // One resource per array over the nparts slots' rows of this head block;
  // part i is at scalar offset i * G rows.  Lanes past the group read
  // neighbouring rows (or zeros past the range) and store nothing.
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(a.part_o + row0 * D, 0, nparts * G * D * 4, PKV_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rl =
      __builtin_amdgcn_make_buffer_rsrc(a.part_lse + row0, 0, nparts * G * 4, PKV_RSRC_WORD3);
  merge_core<kBf16, D, kMulti, kGroupParts>(a, b, h, gb, nparts, lane, [&](int i, float& l, f32x4 (&v)[O::NV]) {
    l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * n, 4 * G * i, kDeviceScope));
#pragma unroll
    for (int nb = 0; nb < O::NV; ++nb)
      v[nb] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, 4 * (n * D + 16 * nb + 4 * c), 4 * G * D * i, kDeviceScope));
  });
  if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The workgroup merge (one 16-column block, static schedule): part i of the
// pair is chunk first + i, whose wavefront left it in its LDS slot 1 (i = 0:
// the pair starts in that chunk) or 0 (the pair began earlier).
template <bool kBf16, int D, bool kMulti>
__device__ void merge_workgroup(const DecodeArgs& a, const PendingMerges& p, int lane) {
  using O = Ops<kBf16, D>;
  const int c = lane >> 4, n = lane & 15;
  const int cols = a.cols;
  const int nparts = p.wparts;
  merge_core<kBf16, D, kMulti, 0>(a, p.wb, p.wh, 0, nparts, lane, [&](int i, float& l, f32x4 (&v)[O::NV]) {
    if (i < nparts && n < cols) {
      const int slot = (p.wfirst + i - p.wg_first) * 2 + (i == 0 ? 1 : 0);
      const float* so = lds_f32 + p.wg_base + (slot * cols + n) * lds_row(D);
      l = lds_f32[p.wg_base + 2 * kWavesPerGroup * cols * lds_row(D) + slot * cols + n];
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) v[nb] = *reinterpret_cast<const f32x4*>(so + 16 * nb + 4 * c);
    } else {
      l = 0.f;
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) v[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  });
}

// Rows of sequences with no pages when the decode kernel merges its own
// partials (no combine kernel runs for them): zeros for length 0, NaN for an
// invalid length.  One wavefront; the empty sequences are found 64 at a time.
__device__ void write_empty_rows(const DecodeArgs& a, const int32_t* s_prefix, int D, bool bf16, int lane) {
  const size_t row_elems = static_cast<size_t>(a.q_len) * a.n_q * D;   // all rows of one sequence
  for (int b0 = 0; b0 < a.batch; b0 += kWave) {
    const int bl = b0 + lane;
    const bool empty = bl < a.batch && s_prefix[bl + 1] == s_prefix[bl];
    uint64_t mask = __builtin_amdgcn_ballot_w64(empty);
    while (mask != 0) {
      const int b = b0 + __builtin_ctzll(mask);
      mask &= mask - 1;
      const float fill = a.seq_lens[b] == 0 ? 0.f : NAN;
      const size_t base = static_cast<size_t>(b) * row_elems;
      for (size_t e = lane; e < row_elems; e += kWave) {
        if (bf16) static_cast<__bf16*>(a.out)[base + e] = static_cast<__bf16>(fill);
        else static_cast<float*>(a.out)[base + e] = fill;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 8-bit KV cache: uint8 codes u with a scale s and a zero point z per (token,
// KV head), x = s (u - z).  Tile layouts per (page, KV head):
//   K codes [D/16][16 tokens][16]    (lane l of load j reads bytes 1024 j + 16 l)
//   V codes [D][16 tokens]
//   meta    float [4][16 tokens]     (k scale, k zero, v scale, v zero)
// The codes enter fp16 MFMAs as 1024 + u: one byte permute builds two such
// fp16 values (0x64 is the high byte of 1024, whose unit in the last place is
// 1), and the 1024 is folded into the zero point.  Scores are
//   s_t (sum_f (1024 + u_tf) q_f - (1024 + z_t) sum_f q_f),
// and the value sum is sum_t w_t (1024 + u_t) - sum_t w_t (1024 + z_t) with
// w_t = p_t s_t, so no element is dequantized one by one.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
constexpr float kCodeBias = 1024.0f;

// Codes 2e and 2e + 1 of the word as the fp16 pair (1024 + u, 1024 + u').
template <int E>
__device__ inline uint32_t code_pair_f16(uint32_t w) {
  return __builtin_amdgcn_perm(0x64646464u, w, E == 0 ? 0x04010400u : 0x04030402u);
}

template <int D>
struct PageRegsQ8 {
  static constexpr int NK = D / 64;   // 16-byte K loads per lane
  static constexpr int NV = D / 16;   // V words per lane (4 tokens of one feature), four per 16-byte load
  u32x4 k[NK];
  uint32_t v[NV];
  f32x4 ks, kz, vs, vz;               // tokens 4c .. 4c+3
};

// Byte of (feature d, slot s) in an 8-bit V-code tile.  The MFMA's value
// operand puts slots 4c .. 4c+3 of feature 16 nb + n in lane (c, n) =
// 16 c + n; the tile stores those four bytes, for nb = 4 j .. 4 j + 3, as
// the 16 bytes at 1024 j + 16 lane, so a lane reads its V codes with D / 64
// sixteen-byte loads (four-byte loads, one per feature block, gathered
// measurably slower: about 5.3 against 6.3 TB/s for the whole tile stream).
__host__ __device__ constexpr int q8_v_offset(int d, int s) {
  return 1024 * (d >> 6) + 256 * (s >> 2) + 16 * (d & 15) + 4 * ((d >> 4) & 3) + (s & 3);
}
static_assert(q8_v_offset(127, 15) == 2047 && q8_v_offset(63, 15) == 1023 && q8_v_offset(16, 0) == 4 &&
                  q8_v_offset(1, 4) == 272,
              "V-code tile order");

// The 8-bit quantizer of one vector of D features, decided in float32 with
// IEEE division and round-half-to-even: lo = min(min x, 0), hi = max(max x,
// 0), s = (hi - lo) / 255 (1 when hi == lo), z = rint(-lo / s), u =
// clamp(rint(x / s) + z, 0, 255).  q8_params takes the two features this
// lane holds (zeros where it holds none: the range includes 0 anyway) and
// reduces over the wavefront; a minimum and a maximum do not depend on which
// lane holds which feature.  The quantizing append kernel (features lane and
// lane + 64) and the decode kernel's fused append (features 2 lane and
// 2 lane + 1) both use these, so their codes agree bit for bit.
__device__ inline float bf16_bits_to_f32(uint32_t bits) { return __builtin_bit_cast(float, bits << 16); }
// Value of lane i ^ 1, i ^ 2 (within each quad), 7 - i within each half row
// and 15 - i within each row of 16 lanes: DPP moves, no LDS round trip.
template <int kCtrl>
__device__ inline float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror
constexpr int kDppMirror = 0x140;       // row_mirror
// Wave-wide minimum and maximum: within each row by DPP (neighbours, pairs,
// then the mirrored half and row, which after the quad steps hold the other
// quad and the other half), then the four rows' results as scalars.  A
// minimum or maximum does not depend on the order it is taken in.
__device__ inline void wave_min_max(float& lo, float& hi) {
  lo = fminf(lo, dpp_f32<kDppXor1>(lo));
  hi = fmaxf(hi, dpp_f32<kDppXor1>(hi));
  lo = fminf(lo, dpp_f32<kDppXor2>(lo));
  hi = fmaxf(hi, dpp_f32<kDppXor2>(hi));
  lo = fminf(lo, dpp_f32<kDppHalfMirror>(lo));
  hi = fmaxf(hi, dpp_f32<kDppHalfMirror>(hi));
  lo = fminf(lo, dpp_f32<kDppMirror>(lo));
  hi = fmaxf(hi, dpp_f32<kDppMirror>(hi));
  auto lane_f = [](float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  };
  lo = fminf(fminf(lane_f(lo, 0), lane_f(lo, 16)), fminf(lane_f(lo, 32), lane_f(lo, 48)));
  hi = fmaxf(fmaxf(lane_f(hi, 0), lane_f(hi, 16)), fmaxf(lane_f(hi, 32), lane_f(hi, 48)));
}
__device__ inline void q8_params(float x0, float x1, float& sc, float& z) {
  float lo = fminf(fminf(x0, x1), 0.f);
  float hi = fmaxf(fmaxf(x0, x1), 0.f);
  wave_min_max(lo, hi);
  sc = (hi - lo) / 255.0f;
  if (sc == 0.f) sc = 1.0f;
  z = __builtin_rintf(-lo / sc);
}
__device__ inline uint32_t q8_code(float x, float sc, float z) {
  return static_cast<uint32_t>(fminf(fmaxf(__builtin_rintf(x / sc) + z, 0.f), 255.f));
}

// Weights of one page's four tokens in a lane, w = p s rounded to fp16
// (p = 2^(x - m)), added to l, and their correction sum
// sum_t w_t (1024 + z_t), returned.  On a page that some key range cuts
// (`cut`, uniform), masked slots (x = -inf) weigh nothing whatever their
// codes and scales hold (possibly NaN); elsewhere every slot is a key.
__device__ inline float q8_weights(const float (&x)[4], float m, f32x4 vs, f32x4 vz, bool cut, float& l, f16x4& wh) {
  float wz = 0.f;
  if (cut) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(x[i] - m);
      l += p;
      const bool in = x[i] != -INFINITY;
      wh[i] = static_cast<_Float16>(in ? p * vs[i] : 0.f);
      wz += in ? static_cast<float>(wh[i]) * (kCodeBias + vz[i]) : 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(x[i] - m);
      l += p;
      wh[i] = static_cast<_Float16>(p * vs[i]);
      wz += static_cast<float>(wh[i]) * (kCodeBias + vz[i]);
    }
  }
  return wz;
}

// One segment of the 8-bit cache (same role and lane layout as Segment).
template <int D, bool kMulti>
struct SegmentQ8 {
  static constexpr int NQ = D / 32;   // fp16 query registers, one per 32-feature MFMA
  static constexpr int NV = D / 16;
  static constexpr int NK = D / 64;   // 16-byte K code loads per lane
  int b, h, gb, g, hq, len, n_pages, fb, q_len, window, hi, lo;
  bool g_ok, append;
  u32x4 qh[NQ];
  float qsum, m, l, corr;
  f32x4 acc[NV];
  // Fused quantizing append (the segment holding the pair's last page): the
  // new token's slot, where its scales and zero points go, and its bf16
  // features 2 lane and 2 lane + 1 of K and of V (zero past D), loaded with
  // the query rows, whose wait they share.
  int s_new;
  char* meta_h;               // meta of page 0, KV head h
  size_t meta_stride;         // bytes between pages of the meta array
  uint32_t kn2, vn2;

  // Query operand of one bf16 row qb (zeros if !g_ok): MFMA 2j + e takes,
  // in lane (c, n), features 16 (4j + c) + 8e .. +7 of head n: the features
  // the K codes of load j bring to lanes of group c.  Returns the sum of the
  // row's fp16 features (the same fp16 values the MFMAs multiply), the same
  // in every lane of the column.
  __device__ static float load_query(const char* qb, bool g_ok, int c, u32x4 (&qh)[NQ]) {
    fetch_row(qb, c, qh);
    return convert_query(qh, g_ok);
  }
  // The two halves of load_query: the row's bf16 pieces as loaded (into qh),
  // then converted in place (returns the sum).  Split so that a caller can
  // issue other loads between them.
  __device__ static void fetch_row(const char* qb, int c, u32x4 (&qh)[NQ]) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) qh[i] = *reinterpret_cast<const u32x4*>(qb + 128 * (i / 2) + 32 * c + 16 * (i % 2));
  }
  __device__ static float convert_query(u32x4 (&qh)[NQ], bool g_ok) {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const u32x4 t = qh[i];
      f16x8 hv;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float lo = __builtin_bit_cast(float, t[w] << 16);
        const float hi = __builtin_bit_cast(float, t[w] & 0xffff0000u);
        hv[2 * w] = static_cast<_Float16>(lo);
        hv[2 * w + 1] = static_cast<_Float16>(hi);
      }
#pragma unroll
      for (int w = 0; w < 8; ++w) part += static_cast<float>(hv[w]);
      qh[i] = g_ok ? __builtin_bit_cast(u32x4, hv) : u32x4{0u, 0u, 0u, 0u};
    }
    part = g_ok ? part : 0.f;
    float sum = part + __shfl_xor(part, 16);
    sum += __shfl_xor(sum, 32);
    return sum;
  }

  __device__ void begin(const DecodeArgs& a, int b_, int h_, int n_pages_, int fb_, bool ends_pair, int gblk,
                        int lane) {
    const int c = lane >> 4, n = lane & 15;
    b = b_;
    h = h_;
    n_pages = n_pages_;
    fb = fb_;
    gb = gblk;
    g = gblk * 16 + n;                 // column (query token qi, query head gq)
    g_ok = g < a.cols;
    const int qi = kMulti ? g / a.group : 0;
    const int gq = g - qi * a.group;
    hq = h * a.group + gq;
    len = seq_len_of(a, b);
    q_len = kMulti ? a.q_len : 1;
    window = kMulti ? a.window : 0;
    hi = len - q_len + qi + 1;
    lo = window > 0 ? max(0, hi - window) : 0;
    append = !kMulti && a.k_new != nullptr && ends_pair;
    s_new = (len - 1) & (kBlock - 1);
    if (append) {
      const size_t row = (static_cast<size_t>(b) * a.n_kv + h) * D;
      const bool in = 2 * lane < D;
      kn2 = in ? reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.k_new) + row)[lane] : 0u;
      vn2 = in ? reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.v_new) + row)[lane] : 0u;
      meta_h = const_cast<char*>(static_cast<const char*>(a.meta)) + static_cast<size_t>(h) * 4 * kBlock * 4;
      meta_stride = static_cast<size_t>(a.n_kv) * 4 * kBlock * 4;
    }
    const size_t qrow = g_ok ? (static_cast<size_t>(b) * q_len + qi) * a.n_q + hq : 0;
    qsum = load_query(static_cast<const char*>(a.q) + qrow * D * 2, g_ok, c, qh);
    m = kNoKeysMax;
    l = 0.f;
    corr = 0.f;
#pragma unroll
    for (int nb = 0; nb < NV; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The new token's codes as this lane holds them in the page registers (K:
  // the 16 codes of features 16 (4 j + c) .. +15 per load j; V: the code of
  // feature 16 nb + n) and its k scale, k zero, v scale, v zero (meta), from
  // this lane's bf16 features 2 lane and 2 lane + 1 of K (kn2) and V (vn2),
  // zeros past D.  Quantized exactly as the quantizing append kernel does;
  // each lane quantizes its two features and lane permutes move the codes to
  // the lanes that hold them.
  __device__ static void quantize_token(uint32_t kn2, uint32_t vn2, int lane, u32x4 (&kq)[NK], uint32_t (&vq)[NV],
                                        f32x4& meta) {
    const int c = lane >> 4, n = lane & 15;
    const float k0 = bf16_bits_to_f32(kn2 & 0xffffu), k1 = bf16_bits_to_f32(kn2 >> 16);
    const float v0 = bf16_bits_to_f32(vn2 & 0xffffu), v1 = bf16_bits_to_f32(vn2 >> 16);
    float ks, kz, vs, vz;
    q8_params(k0, k1, ks, kz);
    q8_params(v0, v1, vs, vz);
    const uint32_t ck = q8_code(k0, ks, kz) | (q8_code(k1, ks, kz) << 8);   // features 2 lane, 2 lane + 1
    const uint32_t cv = q8_code(v0, vs, vz) | (q8_code(v1, vs, vz) << 8);
    // K: lane 2m holds the codes of features 4m .. 4m + 3 in kd; lane (c, n)
    // needs features 16 (4 j + c) .. +15, m = 4 (4 j + c) + q.
    const uint32_t kd = ck | (static_cast<uint32_t>(__shfl_down(static_cast<int>(ck), 1)) << 16);
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int m0 = 8 * (4 * j + c);
      kq[j] = u32x4{static_cast<uint32_t>(__shfl(static_cast<int>(kd), m0)),
                    static_cast<uint32_t>(__shfl(static_cast<int>(kd), m0 + 2)),
                    static_cast<uint32_t>(__shfl(static_cast<int>(kd), m0 + 4)),
                    static_cast<uint32_t>(__shfl(static_cast<int>(kd), m0 + 6))};
    }
    // V: lane (c, n) needs feature 16 nb + n: byte n % 2 of lane 8 nb + n / 2.
#pragma unroll
    for (int nb = 0; nb < NV; ++nb)
      vq[nb] = (static_cast<uint32_t>(__shfl(static_cast<int>(cv), 8 * nb + (n >> 1))) >> (8 * (n & 1))) & 0xffu;
    meta = f32x4{ks, kz, vs, vz};
  }

  // Puts a token into the page registers at slot s_new: its K codes in the
  // lanes n == s_new, its V codes, scales and zero points in the lanes
  // c == s_new / 4, element s_new % 4.
  __device__ static void patch_token(PageRegsQ8<D>& r, const u32x4 (&kq)[NK], const uint32_t (&vq)[NV], f32x4 meta,
                                     int s_new, int lane) {
    const int c = lane >> 4, n = lane & 15;
    if (n == s_new) {
#pragma unroll
      for (int j = 0; j < NK; ++j) r.k[j] = kq[j];
    }
    const int e = s_new & 3;
    if (c == (s_new >> 2)) {
      const uint32_t keep = ~(0xffu << (8 * e));
#pragma unroll
      for (int nb = 0; nb < NV; ++nb) r.v[nb] = (r.v[nb] & keep) | (vq[nb] << (8 * e));
      // element e of each meta vector, by selects (a runtime vector index
      // would put the page registers on the stack)
      auto put = [e](f32x4 v, float x) {
        return f32x4{e == 0 ? x : v[0], e == 1 ? x : v[1], e == 2 ? x : v[2], e == 3 ? x : v[3]};
      };
      r.ks = put(r.ks, meta[0]);
      r.kz = put(r.kz, meta[1]);
      r.vs = put(r.vs, meta[2]);
      r.vz = put(r.vz, meta[3]);
    }
  }

  // The fused append on the pair's last page: the new token (k_new / v_new,
  // bf16) quantized and put into the page registers; if `store`, handed to
  // `held` for page pg (LDS slot `slot`, or written at once if `now`).  Runs
  // once per pair, off the page loop's common path.
  template <class Held>
  __device__ void append_token(PageRegsQ8<D>& r, Held& t, char* kpool, char* vpool, size_t page_stride, int pg,
                               bool store, int slot, int lane, bool now) const {
    u32x4 kq[NK];
    uint32_t vq[NV];
    f32x4 meta;
    quantize_token(kn2, vn2, lane, kq, vq, meta);
    patch_token(r, kq, vq, meta, s_new, lane);
    if (store) {
      const size_t off = static_cast<size_t>(pg) * page_stride;
      t.take(kq, vq, meta, kpool + off, vpool + off, meta_h + static_cast<size_t>(pg) * meta_stride, s_new, slot,
             lane, now);
    }
  }

  // Writes a token's codes, scales and zero points into slot s_new of one
  // (page, KV head) tile: kbase / vbase / mbase are that tile's K codes, V
  // codes and meta.  K: lanes n == s_new, 16 bytes per load; V: one byte per
  // feature from lanes c == s_new / 4 (at q8_v_offset); meta: lanes 0-3.
  __device__ static void store_codes(const u32x4 (&kq)[NK], const uint32_t (&vq)[NV], f32x4 meta, char* kbase,
                                     char* vbase, char* mbase, int s_new, int lane) {
    const int c = lane >> 4, n = lane & 15;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(kbase, 0, kBlock * D, PKV_RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(vbase, 0, kBlock * D, PKV_RSRC_WORD3);
    if (n == s_new) {
#pragma unroll
      for (int j = 0; j < NK; ++j) __builtin_amdgcn_raw_buffer_store_b128(kq[j], kr, 1024 * j + 16 * lane, 0, 0);
    }
    if (c == (s_new >> 2)) {
#pragma unroll
      for (int nb = 0; nb < NV; ++nb)
        __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(vq[nb]), vr, q8_v_offset(16 * nb + n, s_new), 0, 0);
    }
    if (lane < 4) {
      const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(mbase, 0, 4 * kBlock * 4, PKV_RSRC_WORD3);
      const float v = lane == 0 ? meta[0] : lane == 1 ? meta[1] : lane == 2 ? meta[2] : meta[3];
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), mr, 64 * lane + 4 * s_new, 0, 0);
    }
  }

  __device__ void page(PageRegsQ8<D>& r, int j, float scale_log2, int lane) {
    const int c = lane >> 4;
    const int tok0 = kBlock * ((kMulti ? fb : 0) + j);
    const bool cut = kMulti ? tok0 + kBlock > len - q_len + 1 || (window > 0 && tok0 < len - window)
                            : tok0 + kBlock > len;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PageRegsQ8<D>::NK; ++i) {
      const u32x4 kk = r.k[i];
      const u32x4 a0 = {code_pair_f16<0>(kk.x), code_pair_f16<1>(kk.x), code_pair_f16<0>(kk.y),
                        code_pair_f16<1>(kk.y)};
      const u32x4 a1 = {code_pair_f16<0>(kk.z), code_pair_f16<1>(kk.z), code_pair_f16<0>(kk.w),
                        code_pair_f16<1>(kk.w)};
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a0),
                                                 __builtin_bit_cast(f16x8, qh[2 * i]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a1),
                                                 __builtin_bit_cast(f16x8, qh[2 * i + 1]), s1, 0, 0, 0);
    }
    const f32x4 raw = s0 + s1;   // lane (c, n): tokens 4c + i, head n
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = r.ks[i] * (raw[i] - (kCodeBias + r.kz[i]) * qsum) * scale_log2;
    if (cut) {   // uniform: only pages where some column's key range starts or ends
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tok0 + 4 * c + i;
        const bool in = kMulti ? (t < hi && t >= lo) : t < len;   // hi <= len: slots past the sequence are out too
        x[i] = in ? x[i] : -INFINITY;
      }
    }
    const float pm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__builtin_amdgcn_ballot_w64(pm > m + kLazyRescale) != 0) {
      float cm = fmaxf(pm, __shfl_xor(pm, 16));
      cm = fmaxf(cm, __shfl_xor(cm, 32));
      const float mn = fmaxf(m, cm);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
      corr *= alpha;
#pragma unroll
      for (int nb = 0; nb < NV; ++nb) acc[nb] *= alpha;
      m = mn;
    }
    f16x4 wh;
    const float wz = q8_weights(x, m, r.vs, r.vz, cut, l, wh);
    corr += wz;
#pragma unroll
    for (int nb = 0; nb < NV; ++nb) {
      const u32x2 va = {code_pair_f16<0>(r.v[nb]), code_pair_f16<1>(r.v[nb])};
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, va), wh, acc[nb], 0, 0, 0);
    }
  }

  PKV_INLINE __device__ float normalise(bool bad) {
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    float ct = corr + __shfl_xor(corr, 16);
    ct += __shfl_xor(ct, 32);
    const float inv = bad ? NAN : (!kMulti || lt > 0.f ? 1.0f / lt : 0.f);   // no key seen: zero row, lse -inf
#pragma unroll
    for (int nb = 0; nb < NV; ++nb) acc[nb] = (acc[nb] - ct) * inv;
    return bad ? NAN : (m + __log2f(lt)) * kLn2;
  }
  template <class Pending>
  PKV_INLINE __device__ void finish(const DecodeArgs& a, int seg_start, int chunk, int C, bool bad, int lane,
                         Pending& pending) {
    const float lse = normalise(bad);
    emit_segment<true, D, kMulti>(a, b, h, gb, n_pages, seg_start, chunk, C, acc, lse, lane, pending);
  }
};

// New tokens of the fused append on the 8-bit cache, held back like
// HeldToken's: a slot holds the token's D K codes and D V codes in feature
// order, its scales and zero points, and the K code, V code and meta
// addresses of its tile and its slot in the tile.
template <int D, bool kDefer = true>
struct HeldTokenQ8 {
  using Seg = SegmentQ8<D, false>;
  static constexpr int kCodeWords = D / 4;
  static constexpr int kSlotWords = 2 * kCodeWords + 4 + 8;   // K, V, meta, destination
  static_assert(kSlotWords <= kHeldWords, "a held token fits its LDS slot");
  uint32_t* lds;
  uint32_t mask = 0;

  __device__ void store_slot(int i, int lane) {
    mask &= ~(1u << i);
    const int c = lane >> 4, n = lane & 15;
    const uint32_t* w = lds + i * kSlotWords;
    u32x4 kq[Seg::NK];
    uint32_t vq[Seg::NV];
#pragma unroll
    for (int j = 0; j < Seg::NK; ++j) kq[j] = reinterpret_cast<const u32x4*>(w)[4 * j + c];
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(w + kCodeWords);
#pragma unroll
    for (int nb = 0; nb < Seg::NV; ++nb) vq[nb] = vb[16 * nb + n];
    const f32x4 meta = *reinterpret_cast<const f32x4*>(w + 2 * kCodeWords);
    const uint32_t* d = w + 2 * kCodeWords + 4;
    auto u = [](uint32_t x) { return static_cast<uint64_t>(static_cast<uint32_t>(uni(static_cast<int>(x)))); };
    char* kb = reinterpret_cast<char*>((u(d[1]) << 32) | u(d[0]));
    char* vb2 = reinterpret_cast<char*>((u(d[3]) << 32) | u(d[2]));
    char* mb = reinterpret_cast<char*>((u(d[5]) << 32) | u(d[4]));
    Seg::store_codes(kq, vq, meta, kb, vb2, mb, uni(static_cast<int>(d[6])), lane);
  }

  // kq / vq in the lane layout of SegmentQ8::append_token.
  __device__ void take(const u32x4 (&kq)[Seg::NK], const uint32_t (&vq)[Seg::NV], f32x4 meta, char* kbase,
                       char* vbase, char* mbase, int s_new, int slot, int lane, bool now) {
    if (!kDefer || now) {
      Seg::store_codes(kq, vq, meta, kbase, vbase, mbase, s_new, lane);
      return;
    }
    if ((mask >> slot) & 1u) store_slot(slot, lane);
    mask |= 1u << slot;
    const int c = lane >> 4, n = lane & 15;
    uint32_t* w = lds + slot * kSlotWords;
    if (n == 0) {
#pragma unroll
      for (int j = 0; j < Seg::NK; ++j) reinterpret_cast<u32x4*>(w)[4 * j + c] = kq[j];
    }
    if (c == 0) {
      uint8_t* vb = reinterpret_cast<uint8_t*>(w + kCodeWords);
#pragma unroll
      for (int nb = 0; nb < Seg::NV; ++nb) vb[16 * nb + n] = static_cast<uint8_t>(vq[nb]);
    }
    if (lane == 0) {
      *reinterpret_cast<f32x4*>(w + 2 * kCodeWords) = meta;
      const uint64_t kb = reinterpret_cast<uint64_t>(kbase), vb = reinterpret_cast<uint64_t>(vbase),
                     mb = reinterpret_cast<uint64_t>(mbase);
      uint32_t* d = w + 2 * kCodeWords + 4;
      *reinterpret_cast<u32x4*>(d) = u32x4{static_cast<uint32_t>(kb), static_cast<uint32_t>(kb >> 32),
                                           static_cast<uint32_t>(vb), static_cast<uint32_t>(vb >> 32)};
      d[4] = static_cast<uint32_t>(mb);
      d[5] = static_cast<uint32_t>(mb >> 32);
      d[6] = static_cast<uint32_t>(s_new);
    }
  }

  __device__ void store(int lane) {
    if constexpr (kDefer) {
      while (mask != 0) store_slot(__builtin_ctz(mask), lane);
    }
  }
};
static_assert(HeldTokenQ8<128>::kSlotWords == 128 / 2 + 12 && HeldTokenQ8<64>::kSlotWords == 64 / 2 + 12,
              "the host sizes 8-bit token slots as head_dim / 2 + 12 words");

// Position in the flattened (sequence, KV head, page) order of all pages:
// flat index f, sequence b (with pb = pages before b and n = pages of b),
// KV head h, page j of the pair.
template <bool kMulti>
struct FlatCursor {
  int f, b, h, j, n, pb, fb;   // fb: block of the pair's first page (window start; 0 for one query token)
  __device__ static int first_block_of(const DecodeArgs& a, int b) {
    if constexpr (!kMulti) return 0;
    return a.window > 0 ? uni(first_block(seq_len_of(a, b), a.q_len, a.window)) : 0;
  }
  __device__ void seek(const DecodeArgs& a, const int32_t* s_prefix, int f0) {
    f = f0;
    b = uni(find_seq(s_prefix, a.batch, a.n_kv, f0));
    pb = uni(s_prefix[b]);
    n = uni(s_prefix[b + 1]) - pb;
    fb = first_block_of(a, b);
    const int off = f0 - a.n_kv * pb;
    h = off / n;
    j = off - h * n;
  }
  // Next page; must not be called on the last page of all.
  __device__ void next(const DecodeArgs& a, const int32_t* s_prefix) {
    ++f;
    if (++j == n) {
      j = 0;
      if (++h == a.n_kv) {
        h = 0;
        do {
          ++b;
          pb = uni(s_prefix[b]);
          n = uni(s_prefix[b + 1]) - pb;
        } while (n == 0);
        fb = first_block_of(a, b);
      }
    }
  }
};

// At least two wavefronts per SIMD: caps registers at 256 per lane, which the
// bf16 kernels fit without spilling; fp32 at head_dim 128 needs more and runs
// one wavefront per SIMD.
#ifndef PKV_SPLIT_WAVES_PER_EU
#define PKV_SPLIT_WAVES_PER_EU 2
#endif
#ifndef PKV_Q8_WAVES_PER_EU
#define PKV_Q8_WAVES_PER_EU 2
#endif
template <bool kBf16, int D>
constexpr int kSplitWavesPerEu = (kBf16 || D == 64) ? PKV_SPLIT_WAVES_PER_EU : 1;

// Ring depth of the kernels whose sibling wavefronts (one per 16-head block
// of a large group) read the same pages.
#ifndef PKV_GROUPED_DEPTH
#define PKV_GROUPED_DEPTH 2
#endif
#ifndef PKV_GROUPED_WAVES_PER_EU
#define PKV_GROUPED_WAVES_PER_EU 2
#endif
// Cache policies of the split kernel: what one (page, KV head) holds, how a
// wavefront loads it, and the segment type that consumes it.
template <bool kBf16, int D, bool kMulti_>
struct DenseKV {                       // bf16 or fp32 K/V, the q and out dtype; kMulti: q_len > 1 or a window
  static constexpr int kHeadDim = D;
  static constexpr bool kOutBf16 = kBf16;
  static constexpr bool kFusedAppend = true;
  static constexpr bool kMulti = kMulti_;
  static constexpr int kTileK = kBlock * D * Ops<kBf16, D>::ES;
  static constexpr int kWavesPerEu = kSplitWavesPerEu<kBf16, D>;
  static constexpr int kWavesPerEuGrouped = (kBf16 || D == 64) ? PKV_GROUPED_WAVES_PER_EU : 1;
  using Regs = PageRegs<kBf16, D>;
  using Seg = Segment<kBf16, D, kMulti_>;
  template <bool kDefer>
  using Held = HeldToken<kBf16, D, kDefer>;
  template <int kAux>
  __device__ static void load(Regs& r, const DecodeArgs& a, size_t tile, bool on, int lane) {
    const int c = lane >> 4, n = lane & 15;
    const size_t off = tile * kTileK;
    load_page<kBf16, D, kAux>(r, static_cast<const char*>(a.k_pages) + off, static_cast<const char*>(a.v_pages) + off,
                              16u * lane, Ops<kBf16, D>::ES * (n * kBlock + 4 * c), on ? kTileK : 0);
  }
};

template <int D>
struct Q8KV {                          // 8-bit codes + scales; bf16 q and out
  static constexpr int kHeadDim = D;
  static constexpr bool kOutBf16 = true;
  static constexpr bool kFusedAppend = true;    // quantized in the decode kernel
  static constexpr bool kMulti = false;
  static constexpr int kTileK = kBlock * D;        // bytes of one K (or V) code tile
  static constexpr int kMetaBytes = 4 * kBlock * 4;
  static constexpr int kWavesPerEu = PKV_Q8_WAVES_PER_EU;
  static constexpr int kWavesPerEuGrouped = PKV_GROUPED_WAVES_PER_EU;
  using Regs = PageRegsQ8<D>;
  using Seg = SegmentQ8<D, false>;   // one query token, no window
  template <bool kDefer>
  using Held = HeldTokenQ8<D, kDefer>;
  template <int kAux>
  __device__ static void load(Regs& r, const DecodeArgs& a, size_t tile, bool on, int lane) {
    const int c = lane >> 4;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(a.k_pages) + tile * kTileK, 0, on ? kTileK : 0, PKV_RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(a.v_pages) + tile * kTileK, 0, on ? kTileK : 0, PKV_RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(a.meta)) + tile * kMetaBytes, 0, on ? kMetaBytes : 0,
        PKV_RSRC_WORD3);
#pragma unroll
    for (int j = 0; j < Regs::NK; ++j) r.k[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, 1024 * j + 16 * lane, 0, kAux);
#pragma unroll
    for (int j = 0; j < Regs::NV / 4; ++j) {   // V words 4 j .. 4 j + 3 (q8_v_offset)
      const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(vr, 1024 * j + 16 * lane, 0, kAux);
      r.v[4 * j] = w.x;
      r.v[4 * j + 1] = w.y;
      r.v[4 * j + 2] = w.z;
      r.v[4 * j + 3] = w.w;
    }
    r.ks = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(mr, 16 * c, 0, kAux));
    r.kz = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(mr, 64 + 16 * c, 0, kAux));
    r.vs = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(mr, 128 + 16 * c, 0, kAux));
    r.vz = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(mr, 192 + 16 * c, 0, kAux));
  }
};

template <class KV, int kNG>
constexpr int kKernelWavesPerEu = kNG == 1 ? KV::kWavesPerEu : KV::kWavesPerEuGrouped;

// Split-KV decode: one chunk of the flattened (sequence, KV head, page) order
// per kNG wavefronts, each wavefront taking one 16-query-head block of the
// group (kNG = 1 for groups of at most 16; 2 or 4 for larger groups, whose
// sibling wavefronts read the same tiles, the first from HBM and the others
// mostly from the caches).  A loader cursor runs kDepth pages ahead of the
// compute cursor through a ring of kDepth + 1 register buffers, across pair
// boundaries, so the stream of tile loads never drains inside a chunk; the
// compute cursor closes a segment (writes its output rows or partial) and
// opens the next one when the pair changes.  No barrier after the prefix:
// wavefronts without work return early.
//
// kNB = 2 (with kNG = 1, groups of 17 to 32 columns): each wavefront
// computes both 16-column blocks, so a page is loaded once for the whole
// group and its per-page work (page id, loads, masks, cursor) is shared.
// The state of two blocks needs the whole register file: one wavefront per
// SIMD.  Measured on MI355X against two one-block wavefronts per chunk: +8%
// on the GQA layer with 8 query tokens (32 columns); above 32 columns two
// such wavefronts per chunk lost to four one-block ones (the 131072-token
// MQA layer: 1340 vs 1801 GB/s), which keep all four SIMDs of a CU busy on
// one chunk.  Four blocks in one wavefront spill.
template <class KV, int kDepth, int kNG, int kNB = 1>
__global__ void __launch_bounds__(kWave * kWavesPerGroup)
__attribute__((amdgpu_waves_per_eu(kNB > 1 ? 1 : kKernelWavesPerEu<KV, kNG>)))
split_kernel(DecodeArgs a) {
  constexpr int D = KV::kHeadDim;
  constexpr int kTile = KV::kTileK;
  constexpr int kBufs = kDepth + 1;
  using Regs = typename KV::Regs;
  constexpr int kAux = kNG == 1 ? PKV_KV_LOAD_AUX : PKV_KV_LOAD_AUX_GROUPED;
  static_assert(kWavesPerGroup % kNG == 0, "head blocks per chunk divide the workgroup");

  extern __shared__ int32_t smem[];
  int32_t* s_prefix = smem;
  int32_t* s_wsum = smem + a.batch + 1;
  build_prefix(a.seq_lens, a.batch, a.max_blocks, a.q_len, a.window, s_prefix, s_wsum);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uni(threadIdx.x / kWave);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= a.batch; i += blockDim.x) a.prefix[i] = s_prefix[i];
  if (a.counters != nullptr && blockIdx.x == 0 && wave == 0) write_empty_rows(a, s_prefix, D, KV::kOutBf16, lane);
  const int chunk = static_cast<int>(blockIdx.x) * (kWavesPerGroup / kNG) + wave / kNG;
  const int gblk = (wave % kNG) * kNB;
  if (chunk >= a.n_items || gblk * 16 >= a.cols) return;
  const int total = uni(a.n_kv * s_prefix[a.batch]);
  const int C = chunk_pages(total, a.n_items, a.min_chunk);
  const int64_t f64 = static_cast<int64_t>(chunk) * C;
  if (f64 >= total) return;
  const int f0 = static_cast<int>(f64);
  const int cnt = static_cast<int>(min(f64 + C, static_cast<int64_t>(total))) - f0;
  const size_t page_stride = static_cast<size_t>(kTile) * a.n_kv;
  char* kp0 = static_cast<char*>(a.k_pages);
  char* vp0 = static_cast<char*>(a.v_pages);
  auto bt_row = [&](int b) {
    return (const const_i32*)(a.block_table + static_cast<size_t>(b) * a.max_blocks);
  };

  // ---- loader.  Past the chunk's end the loads are issued with an empty
  // range, so every ring step issues the same instructions but nothing is
  // read; a page id outside the pool is never dereferenced either.
  FlatCursor<KV::kMulti> ld;
  ld.seek(a, s_prefix, f0);
  int issued = 0;
  Regs buf[kBufs];
  int page_of[kBufs];   // page id of each buffer (scalar), for the compute side
  auto issue = [&](Regs& r, int& pg_out) {
    const bool in = issued < cnt;
    const int pg = bt_row(ld.b)[ld.fb + ld.j];
    const bool ok = static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_pages);
    KV::template load<kAux>(r, a, static_cast<size_t>(ok ? pg : 0) * a.n_kv + ld.h, in && ok, lane);
    pg_out = pg;
    if (in) {
      ++issued;
      if (issued < cnt) ld.next(a, s_prefix);
    }
  };

  // ---- compute.  seg[i] is head block gblk + i; block 0 carries the new
  // token of a fused append and lists the pairs to merge.
  FlatCursor<KV::kMulti> cp;
  cp.seek(a, s_prefix, f0);
  typename KV::Seg seg[kNB];
  // This wavefront's LDS: held_cap token slots (fused append), then as many
  // result slots (the wavefront's one or two 16-column blocks each).
  const int held_base = held_offset(a.batch) + wave * a.held_wave_words;
  typename KV::template Held<kNG == 1> held;
  held.lds = reinterpret_cast<uint32_t*>(smem + held_base);
  constexpr bool kHoldResults = kNG == 1;
  HeldResults results;
  if constexpr (kHoldResults) {
    if (a.held_res_words > 0) {
      results.cap = a.held_cap;
      results.base = held_base + a.held_cap * a.held_tok_words;
      results.words = a.held_res_words;
    }
  }
  PendingMerges pending, unused;
  constexpr bool kWgMerge = kNG == 1 && kNB == 1;
  if constexpr (kWgMerge) {
    if (a.wg_merge) {
      pending.wg_base = a.wg_lds_offset;
      pending.wg_first = static_cast<int>(blockIdx.x) * kWavesPerGroup;
    }
  }
  bool open = false, bad = false;
  int seg_start = 0;
  // The segment of the compute cursor's pair from the chunk's page p on:
  // query rows (and the new token) requested, state cleared.
  auto open_segment = [&](int p) {
    const bool ends_pair = cp.j + (cnt - p) >= cp.n;
#pragma unroll
    for (int i = 0; i < kNB; ++i)
      if (i == 0 || (gblk + i) * 16 < a.cols) seg[i].begin(a, cp.b, cp.h, cp.n, cp.fb, i == 0 && ends_pair, gblk + i, lane);
    seg_start = a.n_kv * cp.pb + cp.h * cp.n;
    bad = false;
    open = true;
  };
  auto compute = [&](Regs& r, int pg, int p) {
    if (open && (cp.b != seg[0].b || cp.h != seg[0].h)) {
      if (kHoldResults && results.n < results.cap) {
#pragma unroll
        for (int i = 0; i < kNB; ++i)
          if (i == 0 || (gblk + i) * 16 < a.cols) {
            const float lse = seg[i].normalise(bad);
            results.put_block<D>(a, i, seg[i].acc, lse, lane);
          }
        results.commit(seg[0].b, seg[0].h, seg[0].n_pages, seg_start, lane);
      } else {
#pragma unroll
        for (int i = 0; i < kNB; ++i)
          if (i == 0 || (gblk + i) * 16 < a.cols)
            seg[i].finish(a, seg_start, chunk, C, bad, lane, i == 0 ? pending : unused);
      }
      open = false;
    }
    if (!open) open_segment(p);
    const bool ok = static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_pages);
    bad |= !ok;
    // Every head block patches its registers; the first one stores the token:
    // at once on the chunk's last page (nothing follows to hold back), else
    // after its tile stream.  With results held, the token takes the slot
    // its segment's result will take (at once if there is none left);
    // otherwise slot 0, whose previous token is pushed out.
    if constexpr (KV::kFusedAppend) {
      if (seg[0].append && cp.j == cp.n - 1) {
        const bool by_result = kHoldResults && results.cap > 0;
        const int slot = by_result ? results.n : 0;
        const bool now = p == cnt - 1 || (by_result ? results.n >= results.cap : a.held_cap == 0);
        seg[0].append_token(r, held, kp0 + static_cast<size_t>(cp.h) * kTile, vp0 + static_cast<size_t>(cp.h) * kTile,
                            page_stride, pg, ok && gblk == 0, slot, lane, now);
      }
    }
#pragma unroll
    for (int i = 0; i < kNB; ++i)
      if (i == 0 || (gblk + i) * 16 < a.cols) seg[i].page(r, cp.j, a.scale_log2, lane);
  };

  // The first segment's query rows go out before the ring's first tiles:
  // vector memory loads complete in order, so the first page then waits for
  // its own tiles only, not for the whole ring.
  open_segment(0);
#pragma unroll
  for (int s = 0; s < kDepth; ++s) issue(buf[s], page_of[s]);
  // Whole turns of the ring, with the steps past the chunk's end skipped by
  // uniform branches: an early exit from inside the unrolled turn makes the
  // compiler's wait counters assume, at the loop head, that every buffer was
  // just requested, and the ring would drain at every page.
  int p = 0;
  while (p < cnt) {
#pragma unroll
    for (int s = 0; s < kBufs; ++s) {
      // Keep the compiler from sinking these loads below the compute: the
      // requests must be in flight while this page is processed.
      __builtin_amdgcn_sched_barrier(0);
      issue(buf[(s + kDepth) % kBufs], page_of[(s + kDepth) % kBufs]);
      __builtin_amdgcn_sched_barrier(0);
      if (p < cnt) {
        compute(buf[s], page_of[s], p);
        if (p + 1 < cnt) cp.next(a, s_prefix);
      }
      ++p;
    }
  }
  if constexpr (kHoldResults) results.emit_all<KV::kOutBf16, D, KV::kMulti, kNB>(a, gblk, chunk, C, lane, pending, unused);
  if (open) {
#pragma unroll
    for (int i = 0; i < kNB; ++i)
      if (i == 0 || (gblk + i) * 16 < a.cols) seg[i].finish(a, seg_start, chunk, C, bad, lane, i == 0 ? pending : unused);
  }
  // Pairs whose chunks all ran in this workgroup: merged from LDS once every
  // wavefront has left its partials there (wavefronts that returned early
  // are not waited for by the barrier).
  if constexpr (kWgMerge) {
    if (a.wg_merge) {
      __syncthreads();
      if (pending.nw) merge_workgroup<KV::kOutBf16, D, KV::kMulti>(a, pending, lane);
    }
  }
  if (pending.n > 0) {
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      if (i > 0 && (gblk + i) * 16 >= a.cols) continue;
      const int last = arrive(a, pending, gblk + i, lane);
      if (last & 1)
        merge_pair<KV::kOutBf16, D, KV::kMulti>(a, pending.b0, pending.h0, gblk + i, pending.first0, pending.nparts0,
                                                lane);
      if (last & 2)
        merge_pair<KV::kOutBf16, D, KV::kMulti>(a, pending.b1, pending.h1, gblk + i, pending.first1, pending.nparts1,
                                                lane);
    }
  }
  // Last, so that no wait of this wavefront (its loads, the arrival's wait
  // for its partial stores) includes the token's stores.
  if constexpr (KV::kFusedAppend) held.store(lane);
}

// Query tiles wider than the split kernel takes (more than 64 columns per KV
// head: a prefill chunk, or a long drafted run), for pkv_paged_decode_multi.
// There is enough independent work without splitting the keys: one
// wavefront owns a tile of kNB * 16 columns (query tokens x query heads) of
// one (sequence, KV head) and runs the online softmax over every page its
// columns attend, from the first tile's window start to its last query
// token, then writes its output rows; no partials, no merge.  The four
// wavefronts of a workgroup take four adjacent tiles of one (sequence, KV
// head) and read the same pages at about the same time.  Every tile of a
// pair runs on one XCD: the hardware hands workgroup i to XCD i mod 8, so
// workgroup i takes pair 8 * (s / n_wg) + i mod 8 (s = i / 8, n_wg
// workgroups per pair), and the pair's K/V are read from HBM about once,
// then served by that XCD's L2.
//
// The page step is arranged for the matrix cores: the score products of
// every block first, then masks (only on pages where some column's range
// [lo, hi) starts or ends, under one uniform branch), then the
// exponentials and the PV products, all in one basic block.  A column's
// running maximum is set from the first page where it sees a key (its sum
// and accumulator are still zero then, so nothing is rescaled) and is not
// raised afterwards: later scores may exceed it by up to kPrefillHeadroom
// (log2 units), so the exponentials stay <= 2^64, far inside the fp32 and
// bf16 range, and the accumulators are touched only by the matrix cores.
// If a score ever exceeds that (scores of very different sizes in one
// tile), the tile is redone exactly: one pass for every column's true
// maximum, then the accumulation again from zero with that maximum fixed.
constexpr float kPrefillHeadroom = 64.0f;

// Largest of four scores with two v_max3_f32.  fmaxf on values that cross a
// branch (the masked and unmasked pages) makes the compiler quiet each
// input first (one extra move per value), in case it is a signalling NaN;
// scores come from multiplications and selects and never are one.
__device__ inline float max4_scores(float a, float b, float c, float d) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(r), "v"(d));
  return r;
}

template <bool kBf16, int D, int kNB>
struct PrefillTile {
  using O = Ops<kBf16, D>;
  u32x4 q[kNB][O::NK];
  int hi[kNB], lo[kNB];      // keys [lo, hi) of this lane's column
  float m[kNB];
  // m + kPrefillHeadroom, the score above which a page overruns the column
  // (+inf while the column has no maximum yet); settled (wave-uniform): every
  // column of the wavefront has its maximum, so pages skip the first-keys test.
  float mlim[kNB];
  bool settled;
  // Sums of the weights.  bf16: accumulated by the matrix core as the
  // product of an all-ones operand with the same rounded weights the PV
  // product takes, so every element holds its column's sum over all tokens
  // (and the weights are converted to bf16 in pairs, with nothing to unpack
  // for a vector-unit sum).  fp32: element 0 holds this lane's sum over its
  // four tokens.
  f32x4 lsum[kNB];
  f32x4 acc[kNB][O::NV];

  __device__ void clear_sums() {
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      lsum[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) acc[k][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __device__ void reset() {
#pragma unroll
    for (int k = 0; k < kNB; ++k) m[k] = kNoKeysMax;
    set_limits();
    clear_sums();
  }
  // mlim and settled from the current maxima.
  __device__ void set_limits() {
    bool unset = false;
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      mlim[k] = m[k] == kNoKeysMax ? INFINITY : m[k] + kPrefillHeadroom;
      unset |= m[k] == kNoKeysMax;
    }
    settled = __builtin_amdgcn_ballot_w64(unset) == 0;
  }
  // Column k's sum of weights (the same in every lane of the column).
  __device__ float col_sum(int k) const {
    if constexpr (kBf16) {
      return lsum[k][0];
    } else {
      float lt = lsum[k][0] + __shfl_xor(lsum[k][0], 16);
      return lt + __shfl_xor(lt, 32);
    }
  }

  // Scores of page r in log2 units, masked to each column's key range when
  // `cut`; pm: this lane's maximum per block.
  __device__ void scores(const PageRegs<kBf16, D>& r, bool cut, int tok0, float scale_log2, int c,
                         float (&x)[kNB][4], float (&pm)[kNB]) const {
    raw_scores(r, scale_log2, x, pm);
    if (cut) mask_scores(tok0, c, x, pm);
  }
  // The scores without masks, and their maxima.
  __device__ void raw_scores(const PageRegs<kBf16, D>& r, float scale_log2, float (&x)[kNB][4],
                             float (&pm)[kNB]) const {
    f32x4 s[kNB];
#pragma unroll
    for (int k = 0; k < kNB; ++k) s[k] = kNB > 1 ? O::qk1(r.k, q[k]) : O::qk(r.k, q[k]);
#pragma unroll
    for (int k = 0; k < kNB; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[k][i] = s[k][i] * scale_log2;
#pragma unroll
    for (int k = 0; k < kNB; ++k) pm[k] = max4_scores(x[k][0], x[k][1], x[k][2], x[k][3]);
  }
  // Scores outside each column's key range set to -inf, and the maxima again.
  __device__ void mask_scores(int tok0, int c, float (&x)[kNB][4], float (&pm)[kNB]) const {
#pragma unroll
    for (int k = 0; k < kNB; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tok0 + 4 * c + i;
        const bool in = (t < hi[k]) & (t >= lo[k]);
        x[k][i] = in ? x[k][i] : -INFINITY;
      }
#pragma unroll
    for (int k = 0; k < kNB; ++k) pm[k] = max4_scores(x[k][0], x[k][1], x[k][2], x[k][3]);
  }

  // One page of the accumulation.  Returns true (wave-uniform) if some
  // score exceeded its column's maximum by more than kPrefillHeadroom.
  // fixed: the maxima are exact already (the redo pass).
  __device__ bool page(PageRegs<kBf16, D>& r, int valid, bool cut, int tok0, float scale_log2, int c, bool fixed) {
    float x[kNB][4], pm[kNB];
    scores(r, cut, tok0, scale_log2, c, x, pm);
    const bool over = prepare(r, pm, valid, c, fixed);
    finish(r, x);
    return over;
  }

  // The page step's branches, given its (masked) score maxima: values past
  // the length zeroed, overrun test, the maxima of columns seeing their first
  // keys.  Returns true (wave-uniform) on an overrun.
  __device__ bool prepare(PageRegs<kBf16, D>& r, const float (&pm)[kNB], int valid, int c, bool fixed) {
    if (valid < kBlock) {
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) r.v[nb] = O::mask_v(r.v[nb], c, valid);
    }
    bool over = false;
#pragma unroll
    for (int k = 0; k < kNB; ++k) over |= pm[k] > mlim[k];
    if (!settled) {
      bool init = false;
#pragma unroll
      for (int k = 0; k < kNB; ++k) init |= (m[k] == kNoKeysMax) & (pm[k] > kNoKeysMax);
      if (!fixed && __builtin_amdgcn_ballot_w64(init) != 0) {
#pragma unroll
        for (int k = 0; k < kNB; ++k) {
          float cm = fmaxf(pm[k], __shfl_xor(pm[k], 16));
          cm = fmaxf(cm, __shfl_xor(cm, 32));
          m[k] = (m[k] == kNoKeysMax && cm > kNoKeysMax) ? cm : m[k];
        }
        set_limits();
      }
    }
    return __builtin_amdgcn_ballot_w64(over) != 0;
  }

  // The page step's arithmetic, free of branches: weights, PV products, sums.
  __device__ void finish(const PageRegs<kBf16, D>& r, const float (&x)[kNB][4]) {
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[k][i] - m[k]);
      if constexpr (kBf16) {
        constexpr i16x4 kOnes = {0x3f80, 0x3f80, 0x3f80, 0x3f80};   // bf16 1.0
        const i16x4 pk = pack_bf16x4(p[0], p[1], p[2], p[3]);
#pragma unroll
        for (int nb = 0; nb < O::NV; ++nb)
          acc[k][nb] =
              __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, r.v[nb]), pk, acc[k][nb], 0, 0, 0);
        lsum[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kOnes, pk, lsum[k], 0, 0, 0);
      } else {
        float lk = lsum[k][0];
        O::pv(r.v, p, lk, acc[k]);
        lsum[k][0] = lk;
      }
    }
  }

  // bf16: the weights of one page, rounded and packed as the value
  // product's operand (tokens 4c .. 4c + 3 of this lane's column), per block.
  __device__ void weights(const float (&x)[kNB][4], i16x4 (&pk)[kNB]) const {
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[k][i] - m[k]);
      pk[k] = pack_bf16x4(p[0], p[1], p[2], p[3]);
    }
  }
  // bf16: value products and weight sums of two pages a and b in one
  // 16x16x32 product per feature block, which does the work of two 16x16x16
  // ones in the time of one.  The contraction index of a 16x16x32 product
  // runs over eight elements per lane where the 16x16x16 one has four, and
  // the two operands number them alike, so a lane can put page a's four
  // tokens (4c .. 4c + 3) first and page b's second in both operands: its V
  // registers and its weights as they are, with nothing moved between lanes.
  __device__ void pv_pair(const PageRegs<kBf16, D>& ra, const i16x4 (&pa)[kNB], const PageRegs<kBf16, D>& rb,
                          const i16x4 (&pb)[kNB]) {
    constexpr u32x4 kOnes = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      const u32x2 wa = __builtin_bit_cast(u32x2, pa[k]), wb = __builtin_bit_cast(u32x2, pb[k]);
      const bf16x8 w = __builtin_bit_cast(bf16x8, u32x4{wa.x, wa.y, wb.x, wb.y});
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) {
        const u32x4 v = {ra.v[nb].x, ra.v[nb].y, rb.v[nb].x, rb.v[nb].y};
        acc[k][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), w, acc[k][nb], 0, 0, 0);
      }
      lsum[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kOnes), w, lsum[k], 0, 0, 0);
    }
  }
  // bf16: the same for a page without a partner (the second half zero).
  __device__ void pv_last(const PageRegs<kBf16, D>& ra, const i16x4 (&pa)[kNB]) {
    constexpr u32x4 kOnes = {0x3f803f80u, 0x3f803f80u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      const u32x2 wa = __builtin_bit_cast(u32x2, pa[k]);
      const bf16x8 w = __builtin_bit_cast(bf16x8, u32x4{wa.x, wa.y, 0u, 0u});
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) {
        const u32x4 v = {ra.v[nb].x, ra.v[nb].y, 0u, 0u};
        acc[k][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), w, acc[k][nb], 0, 0, 0);
      }
      lsum[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kOnes), w, lsum[k], 0, 0, 0);
    }
  }

  // Exact per-column maximum over page r (the redo pass).
  __device__ void page_max(const PageRegs<kBf16, D>& r, bool cut, int tok0, float scale_log2, int c) {
    float x[kNB][4], pm[kNB];
    scores(r, cut, tok0, scale_log2, c, x, pm);
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      float cm = fmaxf(pm[k], __shfl_xor(pm[k], 16));
      cm = fmaxf(cm, __shfl_xor(cm, 32));
      m[k] = fmaxf(m[k], cm);
    }
  }
};

// PrefillTile's page step on the 8-bit cache (one query token, kNB blocks of
// 16 query heads): the page's codes are turned into fp16 once for all
// blocks, each block's scores take SegmentQ8's zero-point correction, and
// the value operand carries the zero points itself (codes minus zero
// points), so the accumulators hold sum_t w_t (u_t - z_t) directly.
template <int D, int kNB>
struct WideTileQ8 {
  using Seg = SegmentQ8<D, false>;
  static constexpr int NQ = Seg::NQ, NK = Seg::NK, NV = Seg::NV;
  u32x4 q[kNB][NQ];          // the query rows: bf16 as loaded, then fp16 (convert)
  float qsum[kNB];
  bool gok[kNB];
  int hi[kNB], lo[kNB];      // keys [lo, hi) of this lane's column
  float m[kNB], l[kNB];
  float mlim[kNB];           // see PrefillTile
  bool settled;
  f32x4 acc[kNB][NV];

  __device__ void reset() {
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      m[k] = kNoKeysMax;
      l[k] = 0.f;
#pragma unroll
      for (int nb = 0; nb < NV; ++nb) acc[k][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    set_limits();
  }

  __device__ void set_limits() {   // mlim and settled, as in PrefillTile
    bool unset = false;
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      mlim[k] = m[k] == kNoKeysMax ? INFINITY : m[k] + kPrefillHeadroom;
      unset |= m[k] == kNoKeysMax;
    }
    settled = __builtin_amdgcn_ballot_w64(unset) == 0;
  }
  __device__ void clear_sums() {
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      l[k] = 0.f;
#pragma unroll
      for (int nb = 0; nb < NV; ++nb) acc[k][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // Column k's sum of weights: this lane's four tokens' plus the other lane
  // groups'.
  __device__ float col_sum(int k) const {
    const float lt = l[k] + __shfl_xor(l[k], 16);
    return lt + __shfl_xor(lt, 32);
  }

  // The query rows fetched into q (SegmentQ8::fetch_row) converted to fp16
  // in place, with their sums; after the segment's first tile loads, so that
  // the wait for the rows does not hold those loads back.
  __device__ void convert() {
#pragma unroll
    for (int k = 0; k < kNB; ++k) qsum[k] = Seg::convert_query(q[k], gok[k]);
  }

  // Scores of page r in log2 units (-inf outside each column's key range
  // when `cut`); pm: this lane's maximum per block.
  __device__ void scores(const PageRegsQ8<D>& r, bool cut, int tok0, float scale_log2, int c, float (&x)[kNB][4],
                         float (&pm)[kNB]) const {
    u32x4 a0[NK], a1[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const u32x4 kk = r.k[i];
      a0[i] = u32x4{code_pair_f16<0>(kk.x), code_pair_f16<1>(kk.x), code_pair_f16<0>(kk.y), code_pair_f16<1>(kk.y)};
      a1[i] = u32x4{code_pair_f16<0>(kk.z), code_pair_f16<1>(kk.z), code_pair_f16<0>(kk.w), code_pair_f16<1>(kk.w)};
    }
    f32x4 ksl, kzb;   // per token, shared by the blocks: k scale in log2 units, biased k zero
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ksl[i] = r.ks[i] * scale_log2;
      kzb[i] = kCodeBias + r.kz[i];
    }
    // One accumulation chain per block: the blocks are independent, so the
    // matrix core always has work without a second chain and its sum.
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      f32x4 raw = {0.f, 0.f, 0.f, 0.f};   // lane (c, n): tokens 4c + i, head n of block k
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        raw = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a0[i]),
                                                    __builtin_bit_cast(f16x8, q[k][2 * i]), raw, 0, 0, 0);
        raw = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a1[i]),
                                                    __builtin_bit_cast(f16x8, q[k][2 * i + 1]), raw, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) x[k][i] = (raw[i] - kzb[i] * qsum[k]) * ksl[i];
    }
    if (cut) {   // uniform: only pages where some column's key range starts or ends
#pragma unroll
      for (int k = 0; k < kNB; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tok0 + 4 * c + i;
          x[k][i] = ((t < hi[k]) & (t >= lo[k])) ? x[k][i] : -INFINITY;
        }
    }
#pragma unroll
    for (int k = 0; k < kNB; ++k) pm[k] = max4_scores(x[k][0], x[k][1], x[k][2], x[k][3]);
  }

  // One page of the accumulation; returns true (wave-uniform) if some score
  // exceeded its column's maximum by more than kPrefillHeadroom.  fixed: the
  // maxima are exact already (the redo pass).  valid is implied by the key
  // ranges (hi <= the sequence length).
  __device__ bool page(PageRegsQ8<D>& r, int, bool cut, int tok0, float scale_log2, int c, bool fixed) {
    float x[kNB][4], pm[kNB];
    scores(r, cut, tok0, scale_log2, c, x, pm);
    bool over = false;
#pragma unroll
    for (int k = 0; k < kNB; ++k) over |= pm[k] > mlim[k];
    if (!settled) {   // as in PrefillTile::page
      bool init = false;
#pragma unroll
      for (int k = 0; k < kNB; ++k) init |= (m[k] == kNoKeysMax) & (pm[k] > kNoKeysMax);
      if (!fixed && __builtin_amdgcn_ballot_w64(init) != 0) {
#pragma unroll
        for (int k = 0; k < kNB; ++k) {
          float cm = fmaxf(pm[k], __shfl_xor(pm[k], 16));
          cm = fmaxf(cm, __shfl_xor(cm, 32));
          m[k] = (m[k] == kNoKeysMax && cm > kNoKeysMax) ? cm : m[k];
        }
        set_limits();
      }
    }
    // Value operand: each code minus its token's zero point, (1024 + u) -
    // (1024 + z) in fp16, exact (integers in [-255, 255]), once per page for
    // the four blocks; so the accumulators need no zero-point correction.
    // Slots past the key range (cut pages only) may hold NaN zero points:
    // they take 0 (their weights are 0).
    f32x4 vz = r.vz;
    if (cut) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vz[i] = tok0 + 4 * c + i < hi[0] ? vz[i] : 0.f;
    }
    const f16x2 z01 = {static_cast<_Float16>(kCodeBias + vz[0]), static_cast<_Float16>(kCodeBias + vz[1])};
    const f16x2 z23 = {static_cast<_Float16>(kCodeBias + vz[2]), static_cast<_Float16>(kCodeBias + vz[3])};
    u32x2 va[NV];
#pragma unroll
    for (int nb = 0; nb < NV; ++nb)
      va[nb] = u32x2{__builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, code_pair_f16<0>(r.v[nb])) - z01),
                     __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, code_pair_f16<1>(r.v[nb])) - z23)};
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      f16x4 wh;
      (void)q8_weights(x[k], m[k], r.vs, r.vz, cut, l[k], wh);   // its zero-point sum is not needed here
#pragma unroll
      for (int nb = 0; nb < NV; ++nb)
        acc[k][nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, va[nb]), wh, acc[k][nb], 0, 0, 0);
    }
    return __builtin_amdgcn_ballot_w64(over) != 0;
  }

  // Exact per-column maximum over page r (the redo pass).
  __device__ void page_max(const PageRegsQ8<D>& r, bool cut, int tok0, float scale_log2, int c) {
    float x[kNB][4], pm[kNB];
    scores(r, cut, tok0, scale_log2, c, x, pm);
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      float cm = fmaxf(pm[k], __shfl_xor(pm[k], 16));
      cm = fmaxf(cm, __shfl_xor(cm, 32));
      m[k] = fmaxf(m[k], cm);
    }
  }

};

#ifndef PKV_PREFILL_WAVES_PER_EU
#define PKV_PREFILL_WAVES_PER_EU 1
#endif
// bf16 prefill: value products of two pages per 16x16x32 product
// (PrefillTile::pv_pair); 0 keeps one 16x16x16 product per page.
#ifndef PKV_PREFILL_PAIRED
#define PKV_PREFILL_PAIRED 1
#endif
// Largest batch whose sequences the prefill kernel orders longest first.
#ifndef PKV_PREFILL_RANKED_BATCH
#define PKV_PREFILL_RANKED_BATCH 1024
#endif
template <bool kBf16, int D, int kNB, int kDepth>
__global__ void __launch_bounds__(kWave * kWavesPerGroup)
__attribute__((amdgpu_waves_per_eu(PKV_PREFILL_WAVES_PER_EU)))
prefill_kernel(DecodeArgs a, int tiles_per_pair, int wg_per_pair, int n_pair_groups) {
  using O = Ops<kBf16, D>;
  using Regs = PageRegs<kBf16, D>;
  constexpr int kTile = kBlock * D * O::ES;
  constexpr int kBufs = kDepth + 1;
  constexpr int kCols = kNB * 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uni(threadIdx.x / kWave);
  const int i = static_cast<int>(blockIdx.x);
  const int slot = i >> 3;
  const int pg_group = slot / wg_per_pair;
  if (pg_group >= n_pair_groups) return;                // the whole workgroup
  const int pair = pg_group * 8 + (i & 7);
  if (pair >= a.batch * a.n_kv) return;                 // the whole workgroup
  // Longest sequences first: pair index r * n_kv + h is KV head h of the
  // sequence of rank r in decreasing length (ties by index).  Workgroups are
  // dispatched in index order as CUs free up, so the long tiles start first
  // and the short ones fill in behind them instead of leaving a long tail.
  // Each workgroup ranks the lengths in LDS (batches up to kRankedBatch;
  // larger ones keep the sequence order).  Not with a window: a tile then
  // attends at most the window plus its own tokens, so the tiles of long
  // sequences all take about the same time and the ranking would only add
  // its cost.
  constexpr int kRankedBatch = PKV_PREFILL_RANKED_BATCH;
  __shared__ int32_t s_len[kRankedBatch > 0 ? kRankedBatch : 1];
  __shared__ int32_t s_pick;
  const int r = pair / a.n_kv;
  int b = r;
  const bool ranked = a.window == 0 && a.batch <= kRankedBatch;
  if (ranked) {
    for (int t = threadIdx.x; t < a.batch; t += blockDim.x) s_len[t] = seq_len_of(a, t);
    __syncthreads();
    for (int t = threadIdx.x; t < a.batch; t += blockDim.x) {
      const int lt = s_len[t];
      int rank = 0;
      for (int j = 0; j < a.batch; ++j) {
        const int lj = s_len[j];
        rank += (lj > lt) | ((lj == lt) & (j < t));
      }
      if (rank == r) s_pick = t;
    }
    __syncthreads();
    b = uni(s_pick);
  }
  const int h = pair - r * a.n_kv;
  const int tile = (slot - pg_group * wg_per_pair) * kWavesPerGroup + wave;
  if (tile >= tiles_per_pair) return;
  const int g0 = tile * kCols;                          // first column of the tile
  const int len = ranked ? s_len[b] : seq_len_of(a, b);
  const bool len_ok = len >= a.q_len && len <= a.max_blocks * kBlock;
  // Keys the tile's columns attend: from the window start of its first
  // query token to its last query token.
  const int qi0 = g0 / a.group;
  const int qi1 = min(a.q_len - 1, (min(g0 + kCols, a.cols) - 1) / a.group);
  const int hi = len - a.q_len + qi1 + 1;
  const int lo = a.window > 0 ? max(0, len - a.q_len + qi0 + 1 - a.window) : 0;
  const int fb = len_ok ? lo / kBlock : 0;
  const int cnt = len_ok && hi > 0 ? (hi - 1) / kBlock + 1 - fb : 0;
  // The tile's smallest causal bound (its first query token) and largest
  // window start (its last query token): pages wholly inside [lo1, hi0)
  // need no masks.
  const int hi0 = len - a.q_len + qi0 + 1;
  const int lo1 = a.window > 0 ? max(0, hi - a.window) : 0;
  const int c = lane >> 4, n = lane & 15;

  // Query operands and key ranges per block; column g = (query token qi,
  // query head gq); columns past the tile's end hold zeros and write nothing.
  PrefillTile<kBf16, D, kNB> t;
#pragma unroll
  for (int k = 0; k < kNB; ++k) {
    const int g = g0 + 16 * k + n;
    const bool g_ok = g < a.cols;
    const int qi = g / a.group;
    const int hq = h * a.group + (g - qi * a.group);
    const size_t qrow = g_ok ? (static_cast<size_t>(b) * a.q_len + qi) * a.n_q + hq : 0;
    const char* qb = static_cast<const char*>(a.q) + qrow * D * O::ES;
#pragma unroll
    for (int j = 0; j < O::NK; ++j) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qb + 16 * (4 * j + c));
      t.q[k][j] = g_ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
    t.hi[k] = len - a.q_len + qi + 1;
    t.lo[k] = a.window > 0 ? max(0, t.hi[k] - a.window) : 0;
  }
  const const_i32* row = (const const_i32*)(a.block_table + static_cast<size_t>(b) * a.max_blocks);
  const char* kp0 = static_cast<const char*>(a.k_pages);
  const char* vp0 = static_cast<const char*>(a.v_pages);
  bool bad = !len_ok;
  auto load = [&](Regs& r, int j) {
    const int pg = j < cnt ? row[fb + j] : -1;
    const bool ok = static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_pages);
    const size_t off = (static_cast<size_t>(ok ? pg : 0) * a.n_kv + h) * kTile;
    load_page<kBf16, D>(r, kp0 + off, vp0 + off, 16u * lane, O::ES * (n * kBlock + 4 * c), ok ? kTile : 0);
    return pg;
  };
  // The accumulation over the tile's pages through a ring kDepth pages
  // deep; returns true if some score overran its column's maximum.
  auto run = [&](bool fixed) {
    Regs buf[kBufs];
    int page_of[kBufs];
    int issued = 0;
    bool overflow = false;
#pragma unroll
    for (int s = 0; s < kDepth; ++s) page_of[s] = load(buf[s], issued++);
    int p = 0;
    while (p < cnt) {
#pragma unroll
      for (int s = 0; s < kBufs; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        page_of[(s + kDepth) % kBufs] = load(buf[(s + kDepth) % kBufs], issued++);
        __builtin_amdgcn_sched_barrier(0);
        if (p < cnt) {
          bad |= static_cast<unsigned>(page_of[s]) >= static_cast<unsigned>(a.num_pages);
          const int tok0 = kBlock * (fb + p);
          const bool cut = tok0 + kBlock > hi0 || tok0 < lo1;
          overflow |= t.page(buf[s], len - tok0, cut, tok0, a.scale_log2, c, fixed);
        }
        ++p;
      }
    }
    return overflow;
  };
  // The first pass, software-pipelined: step p runs page p's branches (masks
  // of a cut page, values past the length, first keys, overrun test), then in
  // one basic block the score products of page p + 1 and the weights and PV
  // products of page p, so that the matrix core works on one page while the
  // vector unit finishes the other (one wavefront per SIMD: nothing else
  // would fill either).  Past the last page the next buffer holds zeros from
  // an empty range, and its scores are dropped.
  auto run_pipelined = [&]() {
    Regs buf[kBufs];
    int page_of[kBufs];
    int issued = 0;
    bool overflow = false;
#pragma unroll
    for (int s = 0; s < kDepth; ++s) page_of[s] = load(buf[s], issued++);
    float x[kNB][4], pm[kNB];   // scores of the page computed next, unmasked
    t.raw_scores(buf[0], a.scale_log2, x, pm);
    int p = 0;
    while (p < cnt) {
#pragma unroll
      for (int s = 0; s < kBufs; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        page_of[(s + kDepth) % kBufs] = load(buf[(s + kDepth) % kBufs], issued++);
        __builtin_amdgcn_sched_barrier(0);
        if (p < cnt) {
          bad |= static_cast<unsigned>(page_of[s]) >= static_cast<unsigned>(a.num_pages);
          const int tok0 = kBlock * (fb + p);
          if (tok0 + kBlock > hi0 || tok0 < lo1) t.mask_scores(tok0, c, x, pm);
          overflow |= t.prepare(buf[s], pm, len - tok0, c, false);
          float xn[kNB][4], pmn[kNB];
          t.raw_scores(buf[(s + 1) % kBufs], a.scale_log2, xn, pmn);
          t.finish(buf[s], x);
#pragma unroll
          for (int k = 0; k < kNB; ++k) {
            pm[k] = pmn[k];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[k][i] = xn[k][i];
          }
        }
        ++p;
      }
    }
    return overflow;
  };
  // bf16: the same pipeline with the value products of pages 2i and 2i + 1
  // done together (PrefillTile::pv_pair) in the step of page 2i + 1: page
  // 2i's weights wait in registers and its tile stays in the ring, which
  // holds kDepth + 2 pages (p - 1 .. p + kDepth; one more for an odd depth)
  // so that the load issued in step p overwrites a page whose products are
  // done.  The ring's size is even, so a page's parity is its ring slot's.
  auto run_paired = [&]() {
    constexpr int R = kDepth + 2 + (kDepth % 2);   // even
    Regs buf[R];
    int page_of[R];
    int issued = 0;
    bool overflow = false;
#pragma unroll
    for (int s = 0; s < kDepth; ++s) page_of[s] = load(buf[s], issued++);
    float x[kNB][4], pm[kNB];
    t.raw_scores(buf[0], a.scale_log2, x, pm);
    i16x4 pk_prev[kNB];
    int p = 0;
    while (p < cnt) {
#pragma unroll
      for (int s = 0; s < R; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        page_of[(s + kDepth) % R] = load(buf[(s + kDepth) % R], issued++);
        __builtin_amdgcn_sched_barrier(0);
        if (p < cnt) {
          bad |= static_cast<unsigned>(page_of[s]) >= static_cast<unsigned>(a.num_pages);
          const int tok0 = kBlock * (fb + p);
          if (tok0 + kBlock > hi0 || tok0 < lo1) t.mask_scores(tok0, c, x, pm);
          overflow |= t.prepare(buf[s], pm, len - tok0, c, false);
          float xn[kNB][4], pmn[kNB];
          t.raw_scores(buf[(s + 1) % R], a.scale_log2, xn, pmn);
          i16x4 pk[kNB];
          t.weights(x, pk);
          if (s % 2 == 1) {
            t.pv_pair(buf[s - 1], pk_prev, buf[s], pk);
          } else if (p + 1 < cnt) {
#pragma unroll
            for (int k = 0; k < kNB; ++k) pk_prev[k] = pk[k];
          } else {
            t.pv_last(buf[s], pk);
          }
#pragma unroll
          for (int k = 0; k < kNB; ++k) {
            pm[k] = pmn[k];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[k][i] = xn[k][i];
          }
        }
        ++p;
      }
    }
    return overflow;
  };
  t.reset();
  bool overran;
  if constexpr (kBf16 && kDepth >= 2 && PKV_PREFILL_PAIRED) overran = run_paired();
  else if constexpr (kDepth >= 2) overran = run_pipelined();
  else overran = run(false);
  if (overran) {
    // Rare: redo the tile with every column's exact maximum.
    t.reset();
    for (int p = 0; p < cnt; ++p) {
      Regs r;
      load(r, p);
      const int tok0 = kBlock * (fb + p);
      t.page_max(r, tok0 + kBlock > hi0 || tok0 < lo1, tok0, a.scale_log2, c);
    }
    t.set_limits();
    run(true);
  }
  // A length of 0 gives zero rows (no key seen), an invalid one NaN rows.
  bad = bad && len != 0;
#pragma unroll
  for (int k = 0; k < kNB; ++k) {
    const float lt = t.col_sum(k);
    const float inv = bad ? NAN : (lt > 0.f ? 1.0f / lt : 0.f);
    const int g = g0 + 16 * k + n;
    if (g < a.cols) {
      const size_t orow = out_row<true>(a, b, h, g) * D;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) O::store_out(a.out, orow + 16 * nb + 4 * c, t.acc[k][nb] * inv);
    }
  }
}

// Split-KV decode for 33 to 64 columns per KV head (MQA, or several query
// tokens of a large group), bf16 or (kQ8) the 8-bit cache, whose codes are
// turned into fp16 once per page for all four blocks (WideTileQ8); its
// fused append quantizes the token on the page and stores it at once.  One
// wavefront computes all 64 columns of every page it loads (four 16-column
// blocks, the prefill kernel's page step), so each tile is loaded once per
// workgroup and the per-page work (page id, buffer resources, masks,
// cursors) is done once per page; the kernel with one wavefront per
// 16-column block repeated it four times and streamed a quarter as many
// distinct pages.  A chunk is a workgroup's:
// its four wavefronts take the chunk's pages in turn (wavefront w the pages
// w, w + 4, ...), so they stream four neighbouring pages of the same pair
// at a time.  The four walk the chunk's segments (the runs of pages of one
// (sequence, KV head) pair) together; at the end of each segment each
// leaves its four 16-column blocks of partial softmax state in LDS, and
// after one barrier wavefront j merges block j of the four and writes block
// j of the segment's result: the output rows when the pair lies in this
// chunk, else the chunk's partial,
// merged with the pair's other chunks by the last to arrive (the same
// slots, counters and merge as the other split kernels, per block j).
// Running maxima are set on a column's first keys and not raised in the
// page loop, with the prefill kernel's headroom; a segment that overruns
// it is recomputed by that wavefront with exact maxima before the merge.
// The number of segment ends is the same for the four wavefronts, so they
// pass the same number of workgroup barriers.
template <bool kBf16, int D, bool kMulti, int kDepth, bool kQ8 = false>
__global__ void __launch_bounds__(kWave * kWavesPerGroup)
__attribute__((amdgpu_waves_per_eu(1)))
wide_kernel(DecodeArgs a) {
  static_assert(!kQ8 || (kBf16 && !kMulti), "the 8-bit cache: bf16 q and out, one query token");
  using O = Ops<kBf16, D>;
  using Regs = std::conditional_t<kQ8, PageRegsQ8<D>, PageRegs<kBf16, D>>;
  constexpr int kNB = 4;
  constexpr int NV = D / 16;
  constexpr int kTile = kQ8 ? kBlock * D : kBlock * D * O::ES;   // bytes of one K (or V) tile
  constexpr int kMetaTile = 4 * kBlock * 4;                       // 8-bit cache: meta of one tile
  constexpr int kBufs = kDepth + 1;
  constexpr int kRow = lds_row(D);
  constexpr int kSlotWords = 16 * kRow + 32;   // one block of one wavefront: rows [16][kRow], maxima [16], sums [16]
  extern __shared__ int32_t smem[];
  int32_t* s_prefix = smem;
  build_prefix(a.seq_lens, a.batch, a.max_blocks, a.q_len, a.window, s_prefix, smem + a.batch + 1);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uni(threadIdx.x / kWave);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= a.batch; i += blockDim.x) a.prefix[i] = s_prefix[i];
  if (a.counters != nullptr && blockIdx.x == 0 && wave == 0) write_empty_rows(a, s_prefix, D, kBf16, lane);
  const int chunk = static_cast<int>(blockIdx.x);
  if (chunk >= a.n_items) return;                       // the whole workgroup
  const int total = uni(a.n_kv * s_prefix[a.batch]);
  const int C = chunk_pages(total, a.n_items, a.min_chunk);
  const int64_t f64 = static_cast<int64_t>(chunk) * C;
  if (f64 >= total) return;                             // the whole workgroup
  const int f0 = static_cast<int>(f64);
  const int fend = static_cast<int>(min(f64 + C, static_cast<int64_t>(total)));
  const int c = lane >> 4, n = lane & 15;
  float* mlds = reinterpret_cast<float*>(smem) + a.wg_lds_offset;
  const size_t page_stride = static_cast<size_t>(kTile) * a.n_kv;
  char* kp0 = static_cast<char*>(a.k_pages);
  char* vp0 = static_cast<char*>(a.v_pages);
  auto bt_row = [&](int b) { return (const const_i32*)(a.block_table + static_cast<size_t>(b) * a.max_blocks); };

  // ---- segments of the chunk (the same walk in every wavefront)
  FlatCursor<kMulti> sg;
  sg.seek(a, s_prefix, f0);
  int seg_start = 0, seg_hi = 0, len = 0;              // pair's first flat page; end of the segment in the chunk
  std::conditional_t<kQ8, WideTileQ8<D, kNB>, PrefillTile<kBf16, D, kNB>> t;
  bool bad = false, overflow = false;
  PendingMerges pending;
  // A segment's bounds (scalar), then its query operands and state.  The
  // query rows are requested before the segment's first tiles: vector memory
  // loads complete in order, so the first page waits for its own tiles only,
  // not for the whole ring.
  auto bounds = [&]() {
    seg_start = a.n_kv * sg.pb + sg.h * sg.n;
    seg_hi = min(seg_start + sg.n, fend);
    len = seq_len_of(a, sg.b);
  };
  auto open = [&]() {
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      const int g = 16 * k + n;
      const bool g_ok = g < a.cols;
      const int qi = kMulti ? g / a.group : 0;
      const int hq = sg.h * a.group + (g - qi * a.group);
      const int ql = kMulti ? a.q_len : 1;
      const size_t qrow = g_ok ? (static_cast<size_t>(sg.b) * ql + qi) * a.n_q + hq : 0;
      const char* qb = static_cast<const char*>(a.q) + qrow * D * O::ES;
      if constexpr (kQ8) {   // converted after the first tile loads (t.convert)
        SegmentQ8<D, false>::fetch_row(qb, c, t.q[k]);
        t.gok[k] = g_ok;
      } else {
#pragma unroll
        for (int j = 0; j < O::NK; ++j) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(qb + 16 * (4 * j + c));
          t.q[k][j] = g_ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
      }
      t.hi[k] = len - ql + qi + 1;
      t.lo[k] = kMulti && a.window > 0 ? max(0, t.hi[k] - a.window) : 0;
    }
    t.reset();
    bad = false;
    overflow = false;
  };
  // Page f of the flattened order, in this segment: its tile id, first
  // token, masks; the fused append's token is put into the registers of the
  // pair's last page and stored to the pool.
  auto page_at = [&](Regs& r, int pg, int f, bool fixed) {
    const int j = f - seg_start;                       // page of the pair
    const int tok0 = kBlock * (sg.fb + j);
    const bool ok = static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_pages);
    bad |= !ok;
    if constexpr (!kMulti) {
      if (kQ8 && a.k_new != nullptr && j == sg.n - 1) {
        if constexpr (kQ8) {   // quantized here and stored at once, like the dense token below
          using Seg = SegmentQ8<D, false>;
          const int s_new = (len - 1) & (kBlock - 1);
          const size_t row = (static_cast<size_t>(sg.b) * a.n_kv + sg.h) * D;
          const bool two = 2 * lane < D;
          const uint32_t kn2 = two ? reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.k_new) + row)[lane] : 0u;
          const uint32_t vn2 = two ? reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.v_new) + row)[lane] : 0u;
          u32x4 kq[Seg::NK];
          uint32_t vq[Seg::NV];
          f32x4 meta;
          Seg::quantize_token(kn2, vn2, lane, kq, vq, meta);
          Seg::patch_token(r, kq, vq, meta, s_new, lane);
          if (ok && !fixed) {
            const size_t tile = static_cast<size_t>(pg) * a.n_kv + sg.h;
            Seg::store_codes(kq, vq, meta, kp0 + tile * kTile, vp0 + tile * kTile,
                             const_cast<char*>(static_cast<const char*>(a.meta)) + tile * kMetaTile, s_new, lane);
          }
        }
      } else if (!kQ8 && a.k_new != nullptr && j == sg.n - 1) {
        const int s_new = (len - 1) & (kBlock - 1);
        const size_t row = (static_cast<size_t>(sg.b) * a.n_kv + sg.h) * D;
        u32x4 kn[O::NK];
        uint32_t vn[O::NV];
        const char* kb = static_cast<const char*>(a.k_new) + row * O::ES;
#pragma unroll
        for (int i = 0; i < O::NK; ++i) kn[i] = *reinterpret_cast<const u32x4*>(kb + 16 * (4 * i + c));
#pragma unroll
        for (int nb = 0; nb < O::NV; ++nb) {
          if constexpr (kBf16) vn[nb] = static_cast<const uint16_t*>(a.v_new)[row + 16 * nb + n];
          else vn[nb] = static_cast<const uint32_t*>(a.v_new)[row + 16 * nb + n];
        }
        if constexpr (!kQ8) {
          if (n == s_new) {
#pragma unroll
            for (int i = 0; i < O::NK; ++i) r.k[i] = kn[i];
          }
          if (c == (s_new >> 2)) {
#pragma unroll
            for (int nb = 0; nb < O::NV; ++nb) r.v[nb] = O::insert_v(r.v[nb], s_new & 3, vn[nb]);
          }
          if (ok && !fixed) {
            const size_t off = static_cast<size_t>(pg) * page_stride + static_cast<size_t>(sg.h) * kTile;
            HeldToken<kBf16, D, false>::store_regs(kn, vn, kp0 + off, vp0 + off, s_new, lane);
          }
        }
      }
    }
    const bool cut = kMulti ? (tok0 + kBlock > len - a.q_len + 1 || (a.window > 0 && tok0 < len - a.window))
                            : tok0 + kBlock > len;
    return t.page(r, len - tok0, cut, tok0, a.scale_log2, c, fixed);
  };
  // The (page pg, KV head h) tile's loads; a page id outside the pool reads
  // nothing.
  auto load_tile = [&](Regs& r, int pg, int h) {
    const bool ok = static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_pages);
    const size_t tile = static_cast<size_t>(ok ? pg : 0) * a.n_kv + h;
    if constexpr (kQ8)
      Q8KV<D>::template load<PKV_KV_LOAD_AUX>(r, a, tile, ok, lane);
    else
      load_page<kBf16, D, PKV_KV_LOAD_AUX>(r, kp0 + tile * kTile, vp0 + tile * kTile, 16u * lane,
                                           O::ES * (n * kBlock + 4 * c), ok ? kTile : 0);
  };
  auto load_flat = [&](Regs& r, int f) {              // page f of this segment, loaded and waited for
    const int pg = bt_row(sg.b)[sg.fb + (f - seg_start)];
    load_tile(r, pg, sg.h);
    return pg;
  };
  // End of a segment: exact redo if it overran, then the four-way merge
  // and block `wave` of the result written out.
  auto close = [&]() {
    if (overflow) {
      const int seg_lo = max(seg_start, f0);
      const int first = seg_lo + ((wave - (seg_lo - f0)) % 4 + 4) % 4;
      t.reset();
      for (int f = first; f < seg_hi; f += 4) {
        Regs r;
        load_flat(r, f);
        const int tok0 = kBlock * (sg.fb + f - seg_start);
        const bool cut = kMulti ? (tok0 + kBlock > len - a.q_len + 1 || (a.window > 0 && tok0 < len - a.window))
                                : tok0 + kBlock > len;
        t.page_max(r, cut, tok0, a.scale_log2, c);
      }
      t.set_limits();
      t.clear_sums();
      for (int f = first; f < seg_hi; f += 4) {
        Regs r;
        const int pg = load_flat(r, f);
        page_at(r, pg, f, true);
      }
    }
    // Every wavefront leaves its four blocks in LDS, then wavefront j merges
    // block j of the four: one barrier to publish, one before the slots are
    // written again.
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      const float lt = t.col_sum(j);
      float* slot = mlds + (wave * kNB + j) * kSlotWords;
#pragma unroll
      for (int nb = 0; nb < NV; ++nb) *reinterpret_cast<f32x4*>(slot + n * kRow + 16 * nb + 4 * c) = t.acc[j][nb];
      if (c == 0) {
        slot[16 * kRow + n] = t.m[j];
        slot[16 * kRow + 16 + n] = bad ? NAN : lt;
      }
    }
    __syncthreads();
    f32x4 res[NV];
    float mw[kWavesPerGroup];
    float mx = kNoKeysMax;
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) {
      mw[w] = mlds[(w * kNB + wave) * kSlotWords + 16 * kRow + n];
      mx = fmaxf(mx, mw[w]);
    }
#pragma unroll
    for (int nb = 0; nb < NV; ++nb) res[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float rl = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) {
      const float* slot = mlds + (w * kNB + wave) * kSlotWords;
      const float e = __builtin_amdgcn_exp2f(mw[w] - mx);
      rl += e * slot[16 * kRow + 16 + n];
#pragma unroll
      for (int nb = 0; nb < NV; ++nb) res[nb] += e * *reinterpret_cast<const f32x4*>(slot + n * kRow + 16 * nb + 4 * c);
    }
    const float rm = mx;
    __syncthreads();
    // Block `wave` of the segment's result (nothing for blocks past the group).
    if (16 * wave < a.cols) {
      const bool nan_row = rl != rl;
      const float inv = nan_row ? NAN : (rl > 0.f ? 1.0f / rl : 0.f);   // no key seen: zero row, lse -inf
#pragma unroll
      for (int nb = 0; nb < NV; ++nb) res[nb] *= inv;
      const float lse = nan_row ? NAN : (rm + __log2f(rl)) * kLn2;
      emit_segment<kBf16, D, kMulti>(a, sg.b, sg.h, wave, sg.n, seg_start, chunk, C, res, lse, lane, pending);
    }
  };

  // ---- segment by segment: this wavefront's pages of the segment (every
  // fourth page of the chunk, from f0 + wave) through a ring kDepth pages
  // deep, then the segment's end.  One copy of each in the code.
  bounds();
  for (;;) {
    const int seg_lo = max(seg_start, f0);
    const int first = seg_lo + ((wave - (seg_lo - f0)) % 4 + 4) % 4;
    const int mine = first < seg_hi ? (seg_hi - first + 3) / 4 : 0;
    const const_i32* row = bt_row(sg.b) + sg.fb + (first - seg_start);
    Regs buf[kBufs];
    int page_of[kBufs];
    int issued = 0;
    auto issue = [&](Regs& r, int& pg_out) {
      const int pg = issued < mine ? row[4 * issued] : -1;
      load_tile(r, pg, sg.h);
      pg_out = pg;
      ++issued;
    };
    open();
#pragma unroll
    for (int s = 0; s < kDepth; ++s) issue(buf[s], page_of[s]);
    if constexpr (kQ8) t.convert();
    int p = 0;
    while (p < mine) {
#pragma unroll
      for (int s = 0; s < kBufs; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        issue(buf[(s + kDepth) % kBufs], page_of[(s + kDepth) % kBufs]);
        __builtin_amdgcn_sched_barrier(0);
        if (p < mine) overflow |= page_at(buf[s], page_of[s], first + 4 * p, false);
        ++p;
      }
    }
    close();                                          // every wavefront closes every segment
    if (seg_hi >= fend) break;
    sg.seek(a, s_prefix, seg_hi);                     // the chunk's next segment
    bounds();
  }
  if (pending.n > 0 && 16 * wave < a.cols) {
    const int last = arrive(a, pending, wave, lane);
    if (last & 1) merge_pair<kBf16, D, kMulti>(a, pending.b0, pending.h0, wave, pending.first0, pending.nparts0, lane);
    if (last & 2) merge_pair<kBf16, D, kMulti>(a, pending.b1, pending.h1, wave, pending.first1, pending.nparts1, lane);
  }
}

// Counts the arrivals of the listed pairs after this wavefront's partial
// stores have completed (one lane per pair, up to 64 atomics in flight
// together), merges the pairs for which it arrived last, and empties the
// list.  kGroupParts: partials per round trip of the merge (0: the default).
template <bool kOutBf16, int D, bool kMulti, int kGroupParts>
__device__ void flush_pending(const DecodeArgs& a, PendingList& pl, int lane) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  for (int base = 0; base < pl.n; base += kWave) {
    const int i = base + lane;
    const bool in = i < pl.n;
    const int4 e = in ? pl.list[i] : make_int4(0, 0, 0, 0);
    int old = -1;
    if (in)
      old = __hip_atomic_fetch_add(merge_counter(a, e.x, e.y, 0), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t last = __builtin_amdgcn_ballot_w64(in && old == e.w - 1);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    while (last != 0) {
      const int k = __builtin_ctzll(last);
      last &= last - 1;
      const int4 m = pl.list[base + k];
      merge_pair<kOutBf16, D, kMulti, kGroupParts>(a, uni(m.x), uni(m.y), 0, uni(m.z), uni(m.w), lane);
    }
  }
  pl.n = 0;
}

// Split-KV decode with a dynamic schedule, for at most 16 columns per KV
// head: one workgroup of four wavefronts per CU, one wavefront per chunk at a
// time.  The chunks are those of split_kernel (fixed by n_items and
// min_chunk), so every partial and every merge is the same whichever
// wavefront computes it, and results stay run-to-run identical; only the
// assignment is dynamic.  Wavefront w starts on chunk w and then takes
// chunks W, W + 1, ... (W wavefronts in the grid) from a counter in the
// workspace, requesting the next one as it starts loading the current one.
// Wavefronts that run faster (CUs differ, and so do XCDs) take more chunks,
// so all of them end at about the same time.  The loader moves from one
// chunk to the next without draining its ring; the compute side follows the
// chunk id each ring buffer carries.  Arrivals of split pairs are counted
// once the wavefront has no more work (or its pending list is full), so no
// wait for its own partial stores stalls the stream of tile loads.
// One wavefront per SIMD is all the grid asks for, so the kernel may use the
// whole register file (512 per lane, accumulation registers included).
template <class KV, int kDepth>
__global__ void __launch_bounds__(kWave * kWavesPerGroup)
__attribute__((amdgpu_waves_per_eu(1)))
dyn_kernel(DecodeArgs a) {
  constexpr int D = KV::kHeadDim;
  constexpr int kTile = KV::kTileK;
  constexpr int kBufs = kDepth + 1;
  using Regs = typename KV::Regs;
  constexpr int kAux = PKV_KV_LOAD_AUX;
  extern __shared__ int32_t smem[];
  int32_t* s_prefix = smem;
  int32_t* s_wsum = smem + a.batch + 1;
  build_prefix(a.seq_lens, a.batch, a.max_blocks, a.q_len, a.window, s_prefix, s_wsum);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uni(threadIdx.x / kWave);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= a.batch; i += blockDim.x) a.prefix[i] = s_prefix[i];
  if (a.counters != nullptr && blockIdx.x == 0 && wave == 0) write_empty_rows(a, s_prefix, D, KV::kOutBf16, lane);
  PendingList pl;
  pl.list = reinterpret_cast<int4*>(smem + dyn_pending_offset(a.batch)) + wave * kMaxPending;

  const int total = uni(a.n_kv * s_prefix[a.batch]);
  const int C = chunk_pages(total, a.n_items, a.min_chunk);
  const int n_chunks = (total + C - 1) / C;
  const int W = static_cast<int>(gridDim.x) * kWavesPerGroup;
  // Every wavefront takes from the counter until it is refused once, so a
  // launch makes max(0, n_chunks - W) + W takes; the wavefront refused by
  // the last of them resets the counter to zero for the next launch.
  const int last_take = max(0, n_chunks - W) + W - 1;
  // A take is one buffer atomic over a 4-byte range: only lane 0's offset
  // is in range, the other lanes' operations are dropped.  No branch on the
  // lane: a lane-0 branch here makes the compiler treat the scalar state
  // merged after it (took, nxt, the cursors) as divergent, keep it in
  // vector registers, and wrap every tile load in a waterfall loop.
  const __amdgpu_buffer_rsrc_t work_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.work, 0, 4, PKV_RSRC_WORD3);
  auto take = [&]() { return __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, work_rsrc, 4u * lane, 0, 0); };
  // nxt: the next chunk once known (kUnknown until then; >= n_chunks once
  // refused).  A take is requested at the first step of a ring turn, just
  // before that step's tile loads, and read at step kDepth of the same turn,
  // after the compute side has waited for those loads: vector memory
  // operations complete in order, so the read never waits, and the take's
  // register never lives across the loop (where copies of it would each
  // wait for every load in flight).
  constexpr int kUnknown = -1;
  int nxt = kUnknown;
  int refused = -1;                     // this wavefront's refused take (-1: still taking)
  bool took = false;
  int tk = 0;                           // lane 0: the take in flight (assigned only at a turn's first step)
  auto resolve_v = [&](int v) {         // a take's value -> nxt
    nxt = W + v;
    if (nxt >= n_chunks) refused = v;
  };
  auto resolve = [&]() {                // the take in flight -> nxt
    resolve_v(uni(tk));
    took = false;
  };
  int lchunk = static_cast<int>(blockIdx.x) * kWavesPerGroup + wave;
  bool lmore = lchunk < n_chunks;
  if (!lmore) {                         // no chunk of its own: one (refused) take
    const int t = take();
    resolve_v(uni(t));
  }

  const size_t page_stride = static_cast<size_t>(kTile) * a.n_kv;
  char* kp0 = static_cast<char*>(a.k_pages);
  char* vp0 = static_cast<char*>(a.v_pages);
  auto bt_row = [&](int b) {
    return (const const_i32*)(a.block_table + static_cast<size_t>(b) * a.max_blocks);
  };

  // ---- loader.  Once it has no chunk left, the loads are issued with an
  // empty range (nothing is read) and the buffers carry chunk -1.
  FlatCursor<KV::kMulti> ld;
  int lcnt = 0, lissued = 0;
  if (lmore) {
    ld.seek(a, s_prefix, lchunk * C);
    lcnt = min(C, total - lchunk * C);
  }
  Regs buf[kBufs];
  int page_of[kBufs];
  int chunk_of[kBufs];
  auto issue = [&](Regs& r, int& pg_out, int& chunk_out) {
    int pg = -1, hh = 0;
    if (lmore) {
      pg = bt_row(ld.b)[ld.fb + ld.j];
      hh = ld.h;
    }
    const bool ok = static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_pages);
    KV::template load<kAux>(r, a, static_cast<size_t>(ok ? pg : 0) * a.n_kv + hh, ok, lane);
    pg_out = pg;
    chunk_out = lmore ? lchunk : -1;
    if (lmore) {
      if (++lissued < lcnt) {
        ld.next(a, s_prefix);
      } else {
        // Chunk done.  The next one is normally known by now (chunks are
        // longer than a ring turn); otherwise its take is read here, which
        // waits for the loads in flight.
        if (nxt == kUnknown) {
          if (took) {
            resolve();
          } else {
            const int t = take();
            resolve_v(uni(t));
          }
        }
        if (nxt < n_chunks) {
          lchunk = nxt;
          nxt = kUnknown;
          lissued = 0;
          ld.seek(a, s_prefix, lchunk * C);
          lcnt = min(C, total - lchunk * C);
        } else {
          lmore = false;
        }
      }
    }
  };

  // ---- compute.
  FlatCursor<KV::kMulti> cp;
  int cchunk = -1, ccnt = 0, cpos = 0;
  typename KV::Seg seg;
  typename KV::template Held<true> held;
  held.lds = reinterpret_cast<uint32_t*>(smem + held_offset(a.batch)) + wave * kHeldWords;
  bool open = false, bad = false;
  int seg_start = 0;
  auto close = [&]() {
    seg.finish(a, seg_start, cchunk, C, bad, lane, pl);
    open = false;
    // A full list is counted and merged here, with one partial per round
    // trip: few registers beside the ring's.
    if (pl.n == kMaxPending) flush_pending<KV::kOutBf16, D, KV::kMulti, 1>(a, pl, lane);
  };
  auto compute = [&](Regs& r, int pg, int ch) {
    if (ch != cchunk) {
      if (open) close();
      cchunk = ch;
      cpos = 0;
      cp.seek(a, s_prefix, ch * C);
      ccnt = min(C, total - ch * C);
    } else if (open && (cp.b != seg.b || cp.h != seg.h)) {
      close();
    }
    if (!open) {
      const bool ends_pair = cp.j + (ccnt - cpos) >= cp.n;
      seg.begin(a, cp.b, cp.h, cp.n, cp.fb, ends_pair, 0, lane);
      seg_start = a.n_kv * cp.pb + cp.h * cp.n;
      bad = false;
      open = true;
    }
    const bool ok = static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_pages);
    bad |= !ok;
    if constexpr (KV::kFusedAppend) {
      if (seg.append && cp.j == cp.n - 1)
        seg.append_token(r, held, kp0 + static_cast<size_t>(cp.h) * kTile, vp0 + static_cast<size_t>(cp.h) * kTile,
                         page_stride, pg, ok, 0, lane, false);
    }
    seg.page(r, cp.j, a.scale_log2, lane);
    if (++cpos < ccnt) cp.next(a, s_prefix);
  };

#pragma unroll
  for (int s = 0; s < kDepth; ++s) issue(buf[s], page_of[s], chunk_of[s]);
  // Whole turns of the ring with uniform guards, as in split_kernel.
  bool more = true;
  while (more) {
#pragma unroll
    for (int s = 0; s < kBufs; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0 && refused < 0 && nxt == kUnknown && !took) {
        tk = take();
        took = true;
      }
      issue(buf[(s + kDepth) % kBufs], page_of[(s + kDepth) % kBufs], chunk_of[(s + kDepth) % kBufs]);
      __builtin_amdgcn_sched_barrier(0);
      if (chunk_of[s] >= 0) compute(buf[s], page_of[s], chunk_of[s]);
      else more = false;
      if (s == kDepth && took) resolve();
    }
  }
  if (took) resolve();   // (not reached: a take is resolved within its turn)
  if (open) close();
  if (pl.n > 0) flush_pending<KV::kOutBf16, D, KV::kMulti, 0>(a, pl, lane);
  if constexpr (KV::kFusedAppend) held.store(lane);   // last: no wait of this wavefront includes it
  if (refused == last_take && lane == 0)
    __hip_atomic_store(a.work, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the partials of one output row (sequence b, query head hq) whose KV
// pair spans several chunks: out = sum_i w_i o_i / sum_i w_i with
// w_i = exp(lse_i - max lse).  One workgroup per (row, slice of F features),
// F = D / n_fs: with few rows (a few long pairs) a row is split into slices
// of down to 32 features so the merge still spreads over the chip; with many
// rows a workgroup takes a whole row.  The 256 threads form 256 / (F / 4)
// partial lanes of F / 4 threads; thread (lane, t) takes features 4t .. 4t+3
// of the slice from every lane-count-th partial and merges them in one pass
// with a running maximum (the log-sum-exp identity applied to its own
// partials), eight partials per round trip; the lanes' (max, sum,
// accumulator) are then merged through LDS by the same identity.  Rows of
// empty sequences become zeros, rows of invalid lengths NaN.  The page prefix
// comes from the workspace, where the split kernel stored it.
constexpr int kCombineMinSlice = 32;   // features per workgroup, at the finest split
template <bool kBf16, int kF>
__global__ void __launch_bounds__(256) combine_kernel(DecodeArgs a, int D) {
  __shared__ f32x4 s_acc[256];
  __shared__ float s_m[256];
  __shared__ float s_den[256];
  const int32_t* s_prefix = a.prefix;   // stored by the split kernel
  const int G = a.cols;                       // partial rows per slot
  // The slice width is a compile-time constant: this kernel is bound by
  // latency, and runtime lane counts cost it about 10 % (measured on MI355X).
  constexpr int F = kF;                       // features of this workgroup
  constexpr int tpp = F / 4;                  // threads per partial
  constexpr int n_lanes = 256 / tpp;          // partials in parallel
  const int n_fs = D / F;
  const int row = static_cast<int>(blockIdx.x) / n_fs;   // (b * q_len + qi) * n_q + hq
  const int f0 = (static_cast<int>(blockIdx.x) - row * n_fs) * F;
  const int b = row / (a.q_len * a.n_q);
  const int bq = row - b * a.q_len * a.n_q;
  const int qi = bq / a.n_q;
  const int hq = bq - qi * a.n_q;
  const int h = hq / a.group;
  const int g = qi * a.group + (hq - h * a.group);   // column
  const int pair = b * a.n_kv + h;
  const int n = s_prefix[b + 1] - s_prefix[b];
  const size_t row0 = static_cast<size_t>(row) * D + f0;
  const int tid = threadIdx.x;
  const int t = tid % tpp;
  const int lane = tid / tpp;
  auto store4 = [&](int d, f32x4 x) {
    if (kBf16) {
      __bf16* o = static_cast<__bf16*>(a.out) + row0 + d;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = static_cast<__bf16>(x[e]);
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row0 + d) = x;
    }
  };
  // With counters on, the decode kernel wrote the empty rows and merged the
  // pairs of at most fuse_max_parts chunks.
  const bool fused = a.counters != nullptr;
  if (n == 0) {
    if (fused) return;
    const float fill = (a.seq_lens[b] == 0) ? 0.f : NAN;
    if (tid < tpp) store4(4 * tid, f32x4{fill, fill, fill, fill});
    return;
  }
  const int total = a.n_kv * s_prefix[a.batch];
  const int C = chunk_pages(total, a.n_items, a.min_chunk);
  const int seg_start = a.n_kv * s_prefix[b] + h * n;
  const int c0 = seg_start / C;
  const int c1 = (seg_start + n - 1) / C;
  if (c0 == c1) return;
  const size_t slot0 = static_cast<size_t>(c0) + pair;
  const int nparts = c1 - c0 + 1;
  if (fused && nparts <= a.fuse_max_parts) return;
  const float* lse = a.part_lse + slot0 * G + g;
  const float* po = a.part_o + (slot0 * G + g) * D + f0 + 4 * t;
  const size_t stride_o = static_cast<size_t>(G) * D;

  // A maximum of -inf (no partial yet, or only empty ones) is replaced by 0
  // in the exponents, so empty partials weigh 0 and a NaN lse stays NaN.
  float m = -INFINITY, den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // Eight partials per round trip: with 32-feature slices, up to 256
  // partials per row cost one trip.  The merge is bound by the latency of
  // reading partials written from other XCDs, not by bandwidth.
  constexpr int kUnroll = 8;
  for (int s0 = lane; s0 < nparts; s0 += kUnroll * n_lanes) {
    float l[kUnroll];
    f32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = s0 + u * n_lanes;
      l[u] = -INFINITY;
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s < nparts) {
        l[u] = lse[static_cast<size_t>(s) * G];
        v[u] = *reinterpret_cast<const f32x4*>(po + static_cast<size_t>(s) * stride_o);
      }
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) mn = fmaxf(mn, l[u]);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float r = __expf(m - ms);
    acc *= r;
    den *= r;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float w = __expf(l[u] - ms);
      acc += w * v[u];
      den += w;
    }
    m = mn;
  }
  s_acc[tid] = acc;
  s_m[tid] = m;
  s_den[tid] = den;
  __syncthreads();
  if (tid < tpp) {
    float mx = -INFINITY;
#pragma unroll
    for (int ln = 0; ln < n_lanes; ++ln) mx = fmaxf(mx, s_m[ln * tpp + tid]);
    const float ms = mx == -INFINITY ? 0.f : mx;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    float dsum = 0.f;
#pragma unroll
    for (int ln = 0; ln < n_lanes; ++ln) {
      const int i = ln * tpp + tid;
      const float w = __expf(s_m[i] - ms);
      num += w * s_acc[i];
      dsum += w * s_den[i];
    }
    store4(4 * tid, num / dsum);
  }
}

// Slices per combine row: rows are split (down to 32 features) only while
// the grid would stay below 512 workgroups, so a few long pairs spread over
// the chip and a large batch keeps one workgroup per row.
inline int combine_slices_log2(int64_t rows, int head_dim) {
  int lg = 0;
  while ((2 << lg) * kCombineMinSlice <= head_dim && rows * (2 << lg) <= 512) ++lg;
  return lg;
}

// kv_append: one wavefront per (sequence, KV head); a bit copy of the new key
// (16-byte pieces) and value (single elements) into slot pos % 16.
template <int ES>
__global__ void __launch_bounds__(256)
append_kernel(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
              const int32_t* block_table, const int32_t* positions, int batch, int n_kv, int D,
              int max_blocks, int num_pages) {
  const int lane = threadIdx.x & (kWave - 1);
  const int pair = blockIdx.x * kWavesPerGroup + threadIdx.x / kWave;
  if (pair >= batch * n_kv) return;
  const int b = pair / n_kv;
  const int h = pair - b * n_kv;
  const int pos = positions[b];
  if (pos < 0 || pos >= max_blocks * kBlock) return;
  const int page = block_table[static_cast<size_t>(b) * max_blocks + pos / kBlock];
  if (page < 0 || page >= num_pages) return;
  const int slot = pos % kBlock;
  constexpr int X = 16 / ES;
  const size_t tile = static_cast<size_t>(page) * n_kv + h;  // (page, head) tile index
  const char* ksrc = static_cast<const char*>(k_new) + static_cast<size_t>(pair) * D * ES;
  char* kdst = static_cast<char*>(k_pages) + tile * kBlock * D * ES;
  for (int i = lane; i < D / X; i += kWave)
    *reinterpret_cast<u32x4*>(kdst + (static_cast<size_t>(i) * kBlock + slot) * 16) =
        *reinterpret_cast<const u32x4*>(ksrc + 16 * i);
  if (ES == 2) {
    const uint16_t* vsrc = static_cast<const uint16_t*>(v_new) + static_cast<size_t>(pair) * D;
    uint16_t* vdst = static_cast<uint16_t*>(v_pages) + tile * kBlock * D;
    for (int d = lane; d < D; d += kWave) vdst[d * kBlock + slot] = vsrc[d];
  } else {
    const uint32_t* vsrc = static_cast<const uint32_t*>(v_new) + static_cast<size_t>(pair) * D;
    uint32_t* vdst = static_cast<uint32_t*>(v_pages) + tile * kBlock * D;
    for (int d = lane; d < D; d += kWave) vdst[d * kBlock + slot] = vsrc[d];
  }
}

// copy_blocks: one wavefront per (pair, KV head) copies the K tile and the V
// tile of page src[i] to page dst[i] (copy-on-write of a shared block), 16
// bytes per lane per instruction.  Pairs with an id outside the pool, or
// src == dst, are skipped.
// Quantizing append (8-bit cache): one wavefront per (sequence, KV head)
// quantizes the new token's K and V vectors (each with its own scale and
// zero point) and writes the codes into slot pos % 16 of page
// block_table[b][pos / 16], and the scales and zero points into that slot's
// meta.  pos = positions[b] - from_lens (from_lens = 1 when given lengths).
// The quantizer is decided in float32 exactly as the oracle's: the range
// includes 0, s = (hi - lo) / 255 (1 if hi == lo), z = rint(-lo / s),
// u = clamp(rint(x / s) + z, 0, 255), with IEEE division and
// round-half-to-even.
template <bool kInBf16>
__global__ void __launch_bounds__(256)
append_q8_kernel(const void* k_new, const void* v_new, uint8_t* k_codes, uint8_t* v_codes, float* meta,
                 const int32_t* block_table, const int32_t* positions, int from_lens, int batch, int n_kv,
                 int D, int max_blocks, int num_pages) {
  const int lane = threadIdx.x & (kWave - 1);
  const int item = blockIdx.x * kWavesPerGroup + threadIdx.x / kWave;
  if (item >= batch * n_kv) return;
  const int b = item / n_kv;
  const int h = item - b * n_kv;
  const int pos = positions[b] - from_lens;
  if (pos < 0 || pos >= max_blocks * kBlock) return;
  const int pg = block_table[static_cast<size_t>(b) * max_blocks + pos / kBlock];
  if (pg < 0 || pg >= num_pages) return;
  const int slot = pos % kBlock;
  const size_t row = (static_cast<size_t>(b) * n_kv + h) * D;
  const size_t tile = static_cast<size_t>(pg) * n_kv + h;
  auto read = [&](const void* src, int d) -> float {
    if (kInBf16) {
      const uint32_t bits = static_cast<const uint16_t*>(src)[row + d];
      return __builtin_bit_cast(float, bits << 16);
    }
    return static_cast<const float*>(src)[row + d];
  };
  const bool two = D > kWave;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const void* src = which == 0 ? k_new : v_new;
    const float x0 = read(src, lane);
    const float x1 = two ? read(src, lane + kWave) : 0.f;
    float sc, z;
    q8_params(x0, x1, sc, z);
    for (int e = 0; e < (two ? 2 : 1); ++e) {
      const int d = lane + e * kWave;
      const uint8_t u = static_cast<uint8_t>(q8_code(e == 0 ? x0 : x1, sc, z));
      if (which == 0)
        k_codes[tile * kBlock * D + static_cast<size_t>(d / 16) * 256 + slot * 16 + d % 16] = u;
      else
        v_codes[tile * kBlock * D + q8_v_offset(d, slot)] = u;
    }
    if (lane == 0) {
      meta[tile * 64 + (2 * which) * kBlock + slot] = sc;
      meta[tile * 64 + (2 * which + 1) * kBlock + slot] = z;
    }
  }
}

__global__ void __launch_bounds__(256)
copy_blocks_kernel(char* k_pages, char* v_pages, const int32_t* src, const int32_t* dst,
                   int n_pairs, int n_kv, int tile_bytes, int num_pages) {
  const int lane = threadIdx.x & (kWave - 1);
  const int item = blockIdx.x * kWavesPerGroup + threadIdx.x / kWave;
  if (item >= n_pairs * n_kv) return;
  const int i = item / n_kv;
  const int h = item - i * n_kv;
  const int s = src[i], d = dst[i];
  if (s < 0 || s >= num_pages || d < 0 || d >= num_pages || s == d) return;
  const size_t so = (static_cast<size_t>(s) * n_kv + h) * tile_bytes;
  const size_t dof = (static_cast<size_t>(d) * n_kv + h) * tile_bytes;
  for (int off = 16 * lane; off < tile_bytes; off += 16 * kWave) {
    *reinterpret_cast<u32x4*>(k_pages + dof + off) = *reinterpret_cast<const u32x4*>(k_pages + so + off);
    *reinterpret_cast<u32x4*>(v_pages + dof + off) = *reinterpret_cast<const u32x4*>(v_pages + so + off);
  }
}

// Gather probe: the decode kernel's tile stream with no arithmetic.  The
// same chunks of the flattened (sequence, KV head, page) order, the same
// page-id reads, the same per-tile buffer loads (cache policy, ring depth,
// whole ring turns), but each tile is only folded into an XOR that keeps
// the loads live.  Its rate is what the memory system sustains for the
// workload's own tile list, the ceiling the decode kernel is held to.
// page_stride / head_stride: bytes between consecutive pages and between
// the KV heads of a page (n_kv tiles and one tile in the library's layout;
// other values model padded pages, or K and V tiles interleaved per head
// when v_pages = k_pages + one tile and head_stride = two tiles).
template <bool kBf16, int D, int kDepth>
__global__ void __launch_bounds__(kWave * kWavesPerGroup)
__attribute__((amdgpu_waves_per_eu(kSplitWavesPerEu<kBf16, D>)))
gather_probe_kernel(DecodeArgs a, size_t page_stride, size_t head_stride, uint32_t* sink) {
  using O = Ops<kBf16, D>;
  constexpr int kTile = kBlock * D * O::ES;
  constexpr int kBufs = kDepth + 1;
  extern __shared__ int32_t smem[];
  int32_t* s_prefix = smem;
  build_prefix(a.seq_lens, a.batch, a.max_blocks, 1, 0, s_prefix, smem + a.batch + 1);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uni(threadIdx.x / kWave);
  const int chunk = static_cast<int>(blockIdx.x) * kWavesPerGroup + wave;
  if (chunk >= a.n_items) return;
  const int total = uni(a.n_kv * s_prefix[a.batch]);
  const int C = chunk_pages(total, a.n_items, a.min_chunk);
  const int64_t f64 = static_cast<int64_t>(chunk) * C;
  uint32_t acc = 0;
  if (f64 < total) {
    const int f0 = static_cast<int>(f64);
    const int cnt = static_cast<int>(min(f64 + C, static_cast<int64_t>(total))) - f0;
    const char* kp0 = static_cast<const char*>(a.k_pages);
    const char* vp0 = static_cast<const char*>(a.v_pages);
    const int c = lane >> 4, n = lane & 15;
    FlatCursor<false> ld;
    ld.seek(a, s_prefix, f0);
    int issued = 0;
    PageRegs<kBf16, D> buf[kBufs];
    auto issue = [&](PageRegs<kBf16, D>& r) {
      const bool in = issued < cnt;
      const int pg = ((const const_i32*)(a.block_table + static_cast<size_t>(ld.b) * a.max_blocks))[ld.j];
      const bool ok = static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_pages);
      const size_t off = static_cast<size_t>(ok ? pg : 0) * page_stride + static_cast<size_t>(ld.h) * head_stride;
      load_page<kBf16, D>(r, kp0 + off, vp0 + off, 16u * lane, O::ES * (n * kBlock + 4 * c), in && ok ? kTile : 0);
      if (in) {
        ++issued;
        if (issued < cnt) ld.next(a, s_prefix);
      }
    };
    auto fold = [&](const PageRegs<kBf16, D>& r) {
#pragma unroll
      for (int i = 0; i < O::NK; ++i) acc ^= r.k[i].x ^ r.k[i].y ^ r.k[i].z ^ r.k[i].w;
#pragma unroll
      for (int nb = 0; nb < O::NV; ++nb) {
        acc ^= r.v[nb].x ^ r.v[nb].y;
        if constexpr (!kBf16) acc ^= r.v[nb].z ^ r.v[nb].w;
      }
    };
#pragma unroll
    for (int s = 0; s < kDepth; ++s) issue(buf[s]);
    int p = 0;
    while (p < cnt) {
#pragma unroll
      for (int s = 0; s < kBufs; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        issue(buf[(s + kDepth) % kBufs]);
        __builtin_amdgcn_sched_barrier(0);
        if (p < cnt) fold(buf[s]);
        ++p;
      }
    }
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), off));
  if (lane == 0) sink[chunk] = acc;
}

// The same probe for the 8-bit cache: the 8-bit decode kernel's chunks,
// page-id reads and per-tile loads (K codes, V codes, meta; Q8KV::load),
// each tile only folded into an XOR.
template <int D, int kDepth>
__global__ void __launch_bounds__(kWave * kWavesPerGroup)
__attribute__((amdgpu_waves_per_eu(Q8KV<D>::kWavesPerEu)))
gather_probe_q8_kernel(DecodeArgs a, uint32_t* sink) {
  using Regs = PageRegsQ8<D>;
  constexpr int kBufs = kDepth + 1;
  extern __shared__ int32_t smem[];
  int32_t* s_prefix = smem;
  build_prefix(a.seq_lens, a.batch, a.max_blocks, 1, 0, s_prefix, smem + a.batch + 1);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uni(threadIdx.x / kWave);
  const int chunk = static_cast<int>(blockIdx.x) * kWavesPerGroup + wave;
  if (chunk >= a.n_items) return;
  const int total = uni(a.n_kv * s_prefix[a.batch]);
  const int C = chunk_pages(total, a.n_items, a.min_chunk);
  const int64_t f64 = static_cast<int64_t>(chunk) * C;
  uint32_t acc = 0;
  if (f64 < total) {
    const int f0 = static_cast<int>(f64);
    const int cnt = static_cast<int>(min(f64 + C, static_cast<int64_t>(total))) - f0;
    FlatCursor<false> ld;
    ld.seek(a, s_prefix, f0);
    int issued = 0;
    Regs buf[kBufs];
    auto issue = [&](Regs& r) {
      const bool in = issued < cnt;
      const int pg = ((const const_i32*)(a.block_table + static_cast<size_t>(ld.b) * a.max_blocks))[ld.j];
      const bool ok = static_cast<unsigned>(pg) < static_cast<unsigned>(a.num_pages);
      Q8KV<D>::template load<PKV_KV_LOAD_AUX>(r, a, static_cast<size_t>(ok ? pg : 0) * a.n_kv + ld.h, in && ok,
                                              lane);
      if (in) {
        ++issued;
        if (issued < cnt) ld.next(a, s_prefix);
      }
    };
    auto fold = [&](const Regs& r) {
#pragma unroll
      for (int i = 0; i < Regs::NK; ++i) acc ^= r.k[i].x ^ r.k[i].y ^ r.k[i].z ^ r.k[i].w;
#pragma unroll
      for (int nb = 0; nb < Regs::NV; ++nb) acc ^= r.v[nb];
      // the meta as float sums (an XOR of their bits let the compiler drop
      // the loads)
      const f32x4 m = r.ks + r.kz + r.vs + r.vz;
      acc ^= __builtin_bit_cast(uint32_t, m[0] + m[1] + m[2] + m[3]);
    };
#pragma unroll
    for (int s = 0; s < kDepth; ++s) issue(buf[s]);
    int p = 0;
    while (p < cnt) {
#pragma unroll
      for (int s = 0; s < kBufs; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        issue(buf[(s + kDepth) % kBufs]);
        __builtin_amdgcn_sched_barrier(0);
        if (p < cnt) fold(buf[s]);
        ++p;
      }
    }
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), off));
  if (lane == 0) sink[chunk] = acc;
}

__global__ void __launch_bounds__(256)
read_probe_kernel(const u32x4* __restrict__ buf, size_t n16, uint32_t* sink) {
  uint32_t x = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
    u32x4 v = __builtin_nontemporal_load(buf + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // Keep the loads live: one word per workgroup, written by the lane holding x.
  x ^= __shfl_xor(x, 1);
  if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

__global__ void __launch_bounds__(256)
copy_probe_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

// Launch-cost probe: a kernel that does nothing but, with `barrier` set, meet
// every other workgroup of the grid once.  The barrier is one arrival counter
// (bar[0]) and a generation word (bar[1]): each workgroup's first lane adds 1
// to the counter; the last to arrive clears it and advances the generation,
// the others poll the generation until it moves.  Only valid in a
// cooperative launch, which guarantees that the whole grid is resident; a
// poll still gives up after spin_limit rounds and counts a timeout in
// bar[2], so every wave ends whatever happens.
__global__ void __launch_bounds__(256) launch_probe_kernel(int* bar, int barrier, int spin_limit) {
  if (!barrier) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int gen = __hip_atomic_load(&bar[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int old = __hip_atomic_fetch_add(&bar[0], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == static_cast<int>(gridDim.x) - 1) {
      __hip_atomic_store(&bar[0], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&bar[1], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      for (int i = 0; __hip_atomic_load(&bar[1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen; ++i) {
        if (i >= spin_limit) {
          __hip_atomic_fetch_add(&bar[2], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Host-side launch helpers.
// ---------------------------------------------------------------------------
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_fail(const char* what, hipError_t e) {
  return fail(PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

struct Resolved {
  int n_items;
  int min_chunk;
  int combine_mode;
  int wpc;
  int schedule;   // PKV_SCHEDULE_STATIC or PKV_SCHEDULE_DYNAMIC
  size_t lds;
};

using SplitFn = void (*)(DecodeArgs);

// The split kernel's LDS: the per-sequence page prefix and the per-wave sums
// used to build it.
size_t split_lds_bytes(int batch) {
  return static_cast<size_t>(held_offset(batch) + kWavesPerGroup * kHeldWords) * sizeof(int32_t);
}

// The dynamic kernel's LDS: the same, then each wavefront's pending list.
size_t dyn_lds_bytes(int batch) {
  return static_cast<size_t>(dyn_pending_offset(batch)) * sizeof(int32_t) +
         static_cast<size_t>(kWavesPerGroup) * kMaxPending * 16;
}

// bf16 tiles are 4 KiB per (page, head) at head_dim 128: two pages ahead fit
// beside the accumulators at two wavefronts per SIMD.  fp32 tiles are twice
// as large, so fp32 keeps one page ahead.
constexpr int kPrefetchPages = PKV_PREFETCH_PAGES;

// Pages ahead in the 8-bit kernel's ring: 3 measured no faster than 2, and
// 4 no longer fits the registers of two wavefronts per SIMD (spills).
#ifndef PKV_Q8_PREFETCH_PAGES
#define PKV_Q8_PREFETCH_PAGES 2
#endif

// Groups of 17 to 32 columns: one wavefront computes both head blocks of a
// chunk, with a ring three pages deep (two for fp32 at head_dim 64, one at 128).
constexpr int kWideDepth = 3;
template <bool kMulti>
SplitFn split_fn_wide(int dtype, int head_dim, bool q8) {
  if (q8)
    return head_dim == 128 ? split_kernel<Q8KV<128>, kWideDepth, 1, 2> : split_kernel<Q8KV<64>, kWideDepth, 1, 2>;
  if (dtype == PKV_BF16)
    return head_dim == 128 ? split_kernel<DenseKV<true, 128, kMulti>, kWideDepth, 1, 2>
                           : split_kernel<DenseKV<true, 64, kMulti>, kWideDepth, 1, 2>;
  return head_dim == 128 ? split_kernel<DenseKV<false, 128, kMulti>, 1, 1, 2>
                         : split_kernel<DenseKV<false, 64, kMulti>, 2, 1, 2>;
}

template <int kNG, bool kMulti>
SplitFn split_fn_ng(int dtype, int head_dim, bool q8) {
  constexpr int kDepth = kNG == 1 ? kPrefetchPages : PKV_GROUPED_DEPTH;
  if (q8)
    return head_dim == 128 ? split_kernel<Q8KV<128>, PKV_Q8_PREFETCH_PAGES, kNG>
                           : split_kernel<Q8KV<64>, PKV_Q8_PREFETCH_PAGES, kNG>;
  if (dtype == PKV_BF16)
    return head_dim == 128 ? split_kernel<DenseKV<true, 128, kMulti>, kDepth, kNG>
                           : split_kernel<DenseKV<true, 64, kMulti>, kDepth, kNG>;
  return head_dim == 128 ? split_kernel<DenseKV<false, 128, kMulti>, 1, kNG>
                         : split_kernel<DenseKV<false, 64, kMulti>, 1, kNG>;
}

template <bool kMulti>
SplitFn dyn_fn(int dtype, int head_dim, bool q8) {
  if (q8)
    return head_dim == 128 ? dyn_kernel<Q8KV<128>, PKV_Q8_PREFETCH_PAGES>
                           : dyn_kernel<Q8KV<64>, PKV_Q8_PREFETCH_PAGES>;
  if (dtype == PKV_BF16)
    return head_dim == 128 ? dyn_kernel<DenseKV<true, 128, kMulti>, kPrefetchPages>
                           : dyn_kernel<DenseKV<true, 64, kMulti>, kPrefetchPages>;
  return head_dim == 128 ? dyn_kernel<DenseKV<false, 128, kMulti>, 1>
                         : dyn_kernel<DenseKV<false, 64, kMulti>, 1>;
}

// cols: MFMA columns per KV head (query tokens x query heads); multi: more
// than one query token or a sliding window (dense caches only).
// 33 to 64 columns per KV head on a bf16 or 8-bit cache: the wide kernel
// (one wavefront per page for all four 16-column blocks, pages of a chunk
// taken in turn by the workgroup's four wavefronts).
#ifndef PKV_WIDE_DEPTH
#define PKV_WIDE_DEPTH 2
#endif
inline bool uses_wide(int dtype, int cols, bool q8) { return (q8 || dtype == PKV_BF16) && cols > 32; }
// Its LDS: the page prefix, then four wavefronts' merge slots of 16 columns.
size_t wide_lds_bytes(int batch, int head_dim) {
  return (static_cast<size_t>(held_offset(batch)) + kWavesPerGroup * 4 * (16 * lds_row(head_dim) + 32)) * sizeof(int32_t);
}

SplitFn split_fn(int dtype, int head_dim, int cols, bool q8, bool multi) {
  if (uses_wide(dtype, cols, q8)) {
    if (q8)
      return head_dim == 128 ? wide_kernel<true, 128, false, PKV_WIDE_DEPTH, true>
                             : wide_kernel<true, 64, false, PKV_WIDE_DEPTH, true>;
    if (multi)
      return head_dim == 128 ? wide_kernel<true, 128, true, PKV_WIDE_DEPTH> : wide_kernel<true, 64, true, PKV_WIDE_DEPTH>;
    return head_dim == 128 ? wide_kernel<true, 128, false, PKV_WIDE_DEPTH> : wide_kernel<true, 64, false, PKV_WIDE_DEPTH>;
  }
  if (cols > 16 && cols <= 32) return multi ? split_fn_wide<true>(dtype, head_dim, q8) : split_fn_wide<false>(dtype, head_dim, q8);
  switch (waves_per_chunk(cols)) {
    case 1: return multi ? split_fn_ng<1, true>(dtype, head_dim, q8) : split_fn_ng<1, false>(dtype, head_dim, q8);
    case 2: return multi ? split_fn_ng<2, true>(dtype, head_dim, q8) : split_fn_ng<2, false>(dtype, head_dim, q8);
    default: return multi ? split_fn_ng<4, true>(dtype, head_dim, q8) : split_fn_ng<4, false>(dtype, head_dim, q8);
  }
}

int device_cus(int* n_cu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail("hipDeviceGetAttribute", e);
  return ok();
}

// Default chunk count of the static schedule.  Kernels with one wavefront
// per chunk: one chunk per wavefront of one workgroup per CU.  A second
// resident workgroup on a CU does not add bandwidth: the CU's first
// workgroup takes nearly all of its memory throughput and the second one
// mostly waits, then finishes late (measured on MI355X: 1024 chunks of 128
// pages beat 2048 of 64 by 5% on the 16 x 4096 MHA layer).  Larger groups
// (several wavefronts per chunk): one chunk per resident group of them.
// Wavefronts per chunk of the kernel that serves cols columns per KV head.
int chunk_waves(int cols) { return cols <= 32 ? 1 : waves_per_chunk(cols); }

int default_items(int dtype, int head_dim, int group, size_t lds, int* out) {
  int n_cu = 0;
  int st = device_cus(&n_cu);
  if (st != PKV_OK) return st;
  if (chunk_waves(group) == 1) {
    *out = n_cu * kWavesPerGroup;
    return ok();
  }
  int per_cu = 0;
  hipError_t e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu,
      reinterpret_cast<const void*>(split_fn(dtype, head_dim, group, dtype == PKV_U8, false)),
      kWave * kWavesPerGroup, lds);
  if (e != hipSuccess) return hip_fail("hipOccupancyMaxActiveBlocksPerMultiprocessor", e);
  if (per_cu < 1) per_cu = 1;
  *out = n_cu * per_cu * (kWavesPerGroup / waves_per_chunk(group));
  return ok();
}

int check_decode_shapes(const char* fn, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t batch, int32_t max_blocks_per_seq,
                        int32_t num_pages, int32_t dtype) {
  std::string f(fn);
  if (dtype != PKV_F32 && dtype != PKV_BF16 && dtype != PKV_U8) return fail(PKV_ERR_UNSUPPORTED, f + ": dtype");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, f + ": head_dim must be 64 or 128");
  if (block_size != kBlock) return fail(PKV_ERR_UNSUPPORTED, f + ": block_size must be 16");
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, f + ": n_q_heads must be a positive multiple of n_kv_heads");
  if (n_q_heads / n_kv_heads > kMaxGroup)
    return fail(PKV_ERR_UNSUPPORTED, f + ": more than 64 query heads per KV head");
  if (batch < 0 || batch > kMaxBatch)
    return fail(PKV_ERR_UNSUPPORTED, f + ": batch must be in [0, 15000]");
  if (max_blocks_per_seq < 1 || num_pages < 1)
    return fail(PKV_ERR_INVALID_ARG, f + ": max_blocks_per_seq and num_pages must be >= 1");
  if (static_cast<int64_t>(batch) * max_blocks_per_seq * n_kv_heads >= (int64_t{1} << 31))
    return fail(PKV_ERR_UNSUPPORTED, f + ": batch * max_blocks_per_seq * n_kv_heads >= 2^31");
  return PKV_OK;
}

int resolve_opts(int32_t dtype, int32_t head_dim, int32_t group, int32_t batch, int32_t max_blocks,
                 int32_t n_kv, const pkv_decode_opts* opts, Resolved* r) {
  r->wpc = chunk_waves(group);
  r->combine_mode = opts ? opts->combine_mode : 0;
  if (r->combine_mode != 0 && r->combine_mode != 1)
    return fail(PKV_ERR_INVALID_ARG, "decode: combine_mode must be 0 or 1");
  const int sched = opts ? opts->schedule : PKV_SCHEDULE_AUTO;
  if (sched != PKV_SCHEDULE_AUTO && sched != PKV_SCHEDULE_STATIC && sched != PKV_SCHEDULE_DYNAMIC)
    return fail(PKV_ERR_INVALID_ARG, "decode: schedule must be 0 (auto), 1 (static) or 2 (dynamic)");
  const bool dyn_ok = group <= 16 && dyn_lds_bytes(batch) <= kMaxLdsBytes;
  if (sched == PKV_SCHEDULE_DYNAMIC && !dyn_ok)
    return fail(PKV_ERR_UNSUPPORTED, "decode: the dynamic schedule takes at most 16 columns per KV head "
                                     "(query tokens x group) and a batch whose page prefix fits its LDS");
  r->schedule = (sched == PKV_SCHEDULE_DYNAMIC) ? PKV_SCHEDULE_DYNAMIC : PKV_SCHEDULE_STATIC;
  const bool dyn = r->schedule == PKV_SCHEDULE_DYNAMIC;
  r->lds = dyn ? dyn_lds_bytes(batch) : uses_wide(dtype, group, dtype == PKV_U8) ? wide_lds_bytes(batch, head_dim)
                                                                             : split_lds_bytes(batch);
  r->min_chunk = (opts && opts->min_chunk_pages > 0) ? opts->min_chunk_pages
                 : dyn                                ? kDynMinChunk
                                                      : default_min_chunk(group, dtype == PKV_U8);
  if (opts && opts->n_items > 0) {
    if (opts->n_items > kMaxItems)
      return fail(PKV_ERR_INVALID_ARG, "decode: n_items above 2^22");
    r->n_items = opts->n_items;
    return PKV_OK;
  }
  int st;
  if (dyn) {
    int n_cu = 0;
    st = device_cus(&n_cu);
    r->n_items = n_cu * kWavesPerGroup * kDynChunksPerWave;
  } else {
    st = default_items(dtype, head_dim, group, r->lds, &r->n_items);
  }
  if (st != PKV_OK) return st;
  // No more chunks than the largest possible cache (every sequence at
  // max_blocks_per_seq pages) has chunks of min_chunk pages.
  const int64_t max_pages = static_cast<int64_t>(batch) * max_blocks * n_kv;
  const int64_t cap = std::max<int64_t>(1, (max_pages + r->min_chunk - 1) / r->min_chunk);
  r->n_items = static_cast<int>(std::min<int64_t>(r->n_items, cap));
  return PKV_OK;
}

// Zero fill of n 32-bit words (the scratch's first use on a device).
__global__ void __launch_bounds__(256) fill_zero_kernel(uint32_t* p, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

// The scratch array's address on the current device.  Set up once per
// device, with that device current: the address comes from
// hipGetSymbolAddress (each GPU holds its own copy of the array at its own
// address), and the array is cleared once by a fill kernel on the caller's
// stream, since the decode's counters must be zero before its first use
// (every call leaves them zero afterwards).  A kernel, not hipMemsetAsync, so
// that a first call made under graph capture records no memset node.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

int scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(PKV_ERR_UNSUPPORTED, "scratch: device index above " + std::to_string(kMaxScratchDevices - 1));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
    if (ptr == nullptr || !aligned(ptr, 256)) return fail(PKV_ERR_HIP, "scratch: unexpected symbol address");
    hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint32_t*>(ptr),
                       kScratchBytes / 4);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("scratch clear launch", e);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

#ifndef PKV_PREFILL_DEPTH
#define PKV_PREFILL_DEPTH 2
#endif
// 16-column blocks (query tokens x query heads of one KV head) per
// wavefront of the prefill kernel, and its ring depth.  Four blocks fit the
// register file (bf16: 256 VGPRs + 192 AGPRs at head_dim 128 with the paired
// value products' ring of four pages, no scratch; one wavefront per SIMD);
// fp32 at head_dim 128 takes two, with one page ahead.
// Two wavefronts of two blocks per SIMD measured 36 % slower, three blocks
// 10 % slower.
#ifndef PKV_PREFILL_BLOCKS
#define PKV_PREFILL_BLOCKS 4
#endif
constexpr int kPrefillBlocks = PKV_PREFILL_BLOCKS;
constexpr int kPrefillDepth = PKV_PREFILL_DEPTH;
inline int prefill_blocks(int dtype, int head_dim) { return dtype == PKV_F32 && head_dim == 128 ? 2 : kPrefillBlocks; }

int launch_prefill(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                   const int32_t* seq_lens, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                   void* out, hipStream_t stream, int32_t batch, int32_t max_blocks, int32_t num_pages,
                   int32_t dtype, int32_t q_len, int32_t window) {
  DecodeArgs a{};
  a.q = q;
  a.k_pages = const_cast<void*>(k_pages);
  a.v_pages = const_cast<void*>(v_pages);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.batch = batch;
  a.n_q = n_q_heads;
  a.n_kv = n_kv_heads;
  a.group = n_q_heads / n_kv_heads;
  a.q_len = q_len;
  a.window = window;
  a.cols = q_len * a.group;
  a.max_blocks = max_blocks;
  a.num_pages = num_pages;
  a.scale_log2 = scale * kLog2e;
  const int tile_cols = prefill_blocks(dtype, head_dim) * 16;
  const int tiles = (a.cols + tile_cols - 1) / tile_cols;
  const int wg_per_pair = (tiles + kWavesPerGroup - 1) / kWavesPerGroup;
  const int64_t pairs = static_cast<int64_t>(batch) * n_kv_heads;
  const int64_t groups = (pairs + 7) / 8;
  const int64_t grid = groups * wg_per_pair * 8;
  if (grid > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_decode_multi: too many query tiles");
  using Fn = void (*)(DecodeArgs, int, int, int);
  const Fn fn = dtype == PKV_BF16
                    ? (head_dim == 128 ? prefill_kernel<true, 128, kPrefillBlocks, kPrefillDepth>
                                       : prefill_kernel<true, 64, kPrefillBlocks, kPrefillDepth>)
                    : (head_dim == 128 ? prefill_kernel<false, 128, 2, 1>
                                       : prefill_kernel<false, 64, kPrefillBlocks, kPrefillDepth>);
  hipLaunchKernelGGL(fn, dim3(static_cast<uint32_t>(grid)), dim3(kWave * kWavesPerGroup), 0, stream, a, tiles,
                     wg_per_pair, static_cast<int>(groups));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("prefill kernel launch", e);
  return ok();
}

int decode_common(bool do_split, bool do_combine, const char* fn, const void* q,
                  const void* k_new, const void* v_new,
                  const void* k_pages, const void* v_pages, const void* meta, const int32_t* block_table,
                  const int32_t* seq_lens, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                  int32_t block_size, float scale, void* out, void* stream, int32_t batch,
                  int32_t max_blocks_per_seq, int32_t num_pages, int32_t dtype, void* workspace,
                  size_t workspace_bytes, const pkv_decode_opts* opts, int32_t q_len = 1,
                  int32_t window = 0, bool use_scratch = false) {
  int st = check_decode_shapes(fn, n_q_heads, n_kv_heads, head_dim, block_size, batch,
                               max_blocks_per_seq, num_pages, dtype);
  if (st != PKV_OK) return st;
  std::string f(fn);
  if (q_len < 1 || window < 0)
    return fail(PKV_ERR_INVALID_ARG, f + ": q_len must be >= 1 and window >= 0");
  // Wide query tiles (more than 64 columns per KV head): the prefill kernel,
  // one call of pkv_paged_decode_multi, dense caches, no workspace.
  const bool wide = static_cast<int64_t>(q_len) * (n_q_heads / n_kv_heads) > kMaxGroup;
  if (wide && (!do_split || !do_combine || dtype == PKV_U8 || use_scratch))
    return fail(PKV_ERR_UNSUPPORTED, f + ": q_len * (n_q_heads / n_kv_heads) above 64 is taken by "
                                         "pkv_paged_decode_multi on a dense cache only");
  if (wide && static_cast<int64_t>(q_len) * n_q_heads > (int64_t{1} << 20))
    return fail(PKV_ERR_UNSUPPORTED, f + ": q_len * n_q_heads above 2^20");
  if (q_len > 1 && k_new != nullptr)
    return fail(PKV_ERR_INVALID_ARG, f + ": the fused append takes one token per sequence");
  if (batch == 0) return ok();
  if (wide) {
    if (!seq_lens || !out || !q || !k_pages || !v_pages || !block_table || !aligned(seq_lens, 4) ||
        !aligned(out, 16) || !aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
        !aligned(block_table, 4))
      return fail(PKV_ERR_INVALID_ARG, f + ": NULL or misaligned q/k_pages/v_pages/block_table/seq_lens/out");
    if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, f + ": scale is not finite");
    return launch_prefill(q, k_pages, v_pages, block_table, seq_lens, n_q_heads, n_kv_heads, head_dim, scale, out,
                          static_cast<hipStream_t>(stream), batch, max_blocks_per_seq, num_pages, dtype, q_len,
                          window);
  }
  if (use_scratch) workspace_bytes = kScratchBytes;   // the device array, resolved after the checks
  if (!seq_lens || !out || (!use_scratch && (!workspace || !aligned(workspace, 256))) || !aligned(seq_lens, 4) ||
      !aligned(out, 16))
    return fail(PKV_ERR_INVALID_ARG, f + ": NULL or misaligned seq_lens/out/workspace");
  if (do_split && (!q || !k_pages || !v_pages || !block_table || !aligned(q, 16) ||
                   !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(block_table, 4)))
    return fail(PKV_ERR_INVALID_ARG, f + ": NULL or misaligned q/k_pages/v_pages/block_table");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, f + ": scale is not finite");
  // PKV_U8: 8-bit cache (codes + per-token scales and zero points), bf16 q and out.
  const bool q8 = dtype == PKV_U8;
  if (do_split && q8 != (meta != nullptr))
    return fail(PKV_ERR_INVALID_ARG, f + (q8 ? ": the 8-bit cache needs its meta array (16-byte aligned)"
                                             : ": this entry point takes the 8-bit cache only with dtype PKV_U8"));
  if (do_split && q8 && !aligned(meta, 16)) return fail(PKV_ERR_INVALID_ARG, f + ": meta must be 16-byte aligned");
  if ((k_new != nullptr) != (v_new != nullptr) ||
      (k_new && (!aligned(k_new, 16) || !aligned(v_new, 4))))
    return fail(PKV_ERR_INVALID_ARG, f + ": k_new/v_new must both be given, 16/4-byte aligned");
  const int group = n_q_heads / n_kv_heads;
  const int cols = q_len * group;   // MFMA columns per KV head: (query token, query head)
  Resolved r;
  st = resolve_opts(dtype, head_dim, cols, batch, max_blocks_per_seq, n_kv_heads, opts, &r);
  if (st != PKV_OK) return st;
  if (do_split && r.lds > (uses_wide(dtype, cols, q8) ? kMaxLdsBytesWide : kMaxLdsBytes))
    return fail(PKV_ERR_UNSUPPORTED, f + ": batch too large for this group size (LDS " +
                                         std::to_string(r.lds) + " bytes)");
  const int64_t need = pkv_decode_workspace_bytes(batch, n_q_heads * q_len, n_kv_heads, head_dim, r.n_items);
  if (need < 0) return static_cast<int>(need);
  if (workspace_bytes < static_cast<size_t>(need))
    return fail(PKV_ERR_WORKSPACE, f + (use_scratch ? ": these shapes need " + std::to_string(need) +
                                                          " bytes of scratch, above the library's fixed " +
                                                          std::to_string(kScratchBytes) + " bytes"
                                                    : ": workspace needs " + std::to_string(need) + " bytes"));
  if (use_scratch) {
    st = scratch_of_current_device(static_cast<hipStream_t>(stream), &workspace);
    if (st != PKV_OK) return st;
  }

  const int64_t slots = decode_slots(batch, n_kv_heads, r.n_items);
  DecodeArgs a;
  a.q = q;
  // The pools are written only when the new token is appended in the same launch.
  a.k_pages = const_cast<void*>(k_pages);
  a.v_pages = const_cast<void*>(v_pages);
  a.k_new = k_new;
  a.v_new = v_new;
  a.meta = meta;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = static_cast<float*>(workspace) + slots * cols * head_dim;
  a.batch = batch;
  a.n_q = n_q_heads;
  a.n_kv = n_kv_heads;
  a.group = group;
  a.q_len = q_len;
  a.window = window;
  a.cols = cols;
  a.max_blocks = max_blocks_per_seq;
  a.num_pages = num_pages;
  a.n_items = r.n_items;
  a.min_chunk = r.min_chunk;
  a.waves_per_chunk = r.wpc;
  a.scale_log2 = scale * kLog2e;
  // Merge in the decode kernel when both halves run in this call; the
  // combine kernel then runs only if some pair may span more than
  // fuse_limit chunks (C >= min_chunk, so a pair of at most
  // max_blocks_per_seq pages spans at most ceil(max_blocks / min_chunk) + 1).
  const bool fuse = do_split && do_combine && r.combine_mode == 0;
  const int64_t max_parts = (static_cast<int64_t>(max_blocks_per_seq) + r.min_chunk - 1) / r.min_chunk + 1;
  // The counters are counted backwards from the workspace's last int32
  // word, which is the dynamic schedule's chunk counter.
  int32_t* tail = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + (workspace_bytes & ~size_t{3})) - 1;
  a.counters = fuse ? tail : nullptr;
  a.fuse_max_parts = fuse_limit(uses_wide(dtype, cols, q8), max_parts);
  a.prefix = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                        decode_prefix_offset(batch, cols, n_kv_heads, head_dim, r.n_items));
  a.work = tail;
  // Split kernel LDS (static schedule; r.lds, checked above, holds the
  // prefix and one token slot per wavefront):
  // - workgroup merges (one wavefront per chunk and one 16-column block,
  //   in-kernel merge on) when their slots fit;
  // - then per wavefront as many slots (up to kMaxHeldSlots) of held tokens
  //   and held results (one or two 16-column blocks) as the rest allows;
  //   the two-block kernel runs one workgroup per CU and may take the CU's
  //   whole LDS for them.
  size_t lds = r.lds;
  a.wg_merge = 0;
  a.wg_lds_offset = 0;
  a.held_cap = 0;
  a.held_tok_words = 0;
  a.held_res_words = 0;
  a.held_wave_words = kHeldWords;
  if (r.schedule == PKV_SCHEDULE_STATIC) {
    const bool one_block = cols <= 16;
    const bool two_blocks = cols > 16 && cols <= 32;   // split_fn: one wavefront per SIMD, both blocks
    size_t wg_words = 0;
    if (fuse && one_block) {
      const size_t wg = static_cast<size_t>(kWavesPerGroup) * 2 * cols * (lds_row(head_dim) + 1);
      if (r.lds + wg * sizeof(float) <= kMaxLdsBytes) wg_words = wg;
    }
    const int es = dtype == PKV_F32 ? 4 : 2;
    // HeldToken::kSlotWords, HeldTokenQ8::kSlotWords
    const int tok = k_new == nullptr ? 0 : q8 ? head_dim / 2 + 12 : head_dim * es / 4 + head_dim + 8;
    int res = one_block || two_blocks ? ((cols * (lds_row(head_dim) + 1) + 3) & ~3) + 4 : 0;
    const size_t budget = two_blocks ? kMaxLdsBytesWide : kMaxLdsBytes;
    const size_t avail = budget / sizeof(int32_t) - held_offset(batch) - wg_words;
    int cap = res > 0 ? static_cast<int>(std::min<size_t>(kMaxHeldSlots, avail / (kWavesPerGroup * (tok + res))))
                      : 0;
    if (cap == 0) {   // no results held: one token slot (fits, see r.lds)
      res = 0;
      cap = tok > 0 ? 1 : 0;
    }
    a.held_cap = cap;
    a.held_tok_words = tok;
    a.held_res_words = res;
    a.held_wave_words = cap * (tok + res);
    const size_t held_end = held_offset(batch) + static_cast<size_t>(kWavesPerGroup) * a.held_wave_words;
    lds = held_end * sizeof(int32_t);
    if (wg_words > 0) {
      a.wg_merge = 1;
      a.wg_lds_offset = static_cast<int32_t>(held_end);
      lds += wg_words * sizeof(float);
    }
    if (uses_wide(dtype, cols, q8)) {   // its own LDS: prefix, then the merge slots
      a.wg_merge = 0;
      a.held_cap = 0;
      a.wg_lds_offset = held_offset(batch);
      lds = r.lds;
    }
  }
  const bool run_combine = do_combine && (!fuse || max_parts > a.fuse_max_parts);
  // One combine workgroup per slice of an output row.
  const int64_t combine_rows = static_cast<int64_t>(batch) * q_len * n_q_heads;
  const int fs_log2 = combine_slices_log2(combine_rows, head_dim);
  const int64_t grid_c = combine_rows << fs_log2;
  if (run_combine && grid_c > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, f + ": too many output rows for the combine kernel");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (do_split) {
    const bool multi = q_len > 1 || window > 0;
    SplitFn fn;
    int grid;
    if (r.schedule == PKV_SCHEDULE_DYNAMIC) {
      // one workgroup per CU, never more than one chunk's worth of wavefronts each
      int n_cu = 0;
      st = device_cus(&n_cu);
      if (st != PKV_OK) return st;
      grid = std::max(1, std::min(n_cu, (r.n_items + kWavesPerGroup - 1) / kWavesPerGroup));
      fn = multi ? dyn_fn<true>(dtype, head_dim, q8) : dyn_fn<false>(dtype, head_dim, q8);
    } else {
      const int chunks_per_group = kWavesPerGroup / r.wpc;
      grid = (r.n_items + chunks_per_group - 1) / chunks_per_group;
      fn = split_fn(dtype, head_dim, cols, q8, multi);
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kWave * kWavesPerGroup), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("split kernel launch", e);
  }
  if (run_combine) {
    using CombineFn = void (*)(DecodeArgs, int);
    const bool f32 = dtype == PKV_F32;
    const int width = head_dim >> fs_log2;   // 32, 64 or 128 features per workgroup
    CombineFn fn_c = width == 32   ? (f32 ? combine_kernel<false, 32> : combine_kernel<true, 32>)
                     : width == 64 ? (f32 ? combine_kernel<false, 64> : combine_kernel<true, 64>)
                                   : (f32 ? combine_kernel<false, 128> : combine_kernel<true, 128>);
    hipLaunchKernelGGL(fn_c, dim3(static_cast<uint32_t>(grid_c)), dim3(256), 0, s, a, head_dim);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("combine kernel launch", e);
  }
  return ok();
}

int append_q8_common(const char* fn, const void* k_new, const void* v_new, void* k_codes, void* v_codes,
                     void* meta, const int32_t* block_table, const int32_t* positions, bool from_lens,
                     int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t max_blocks_per_seq, int32_t num_pages, int32_t dtype, void* stream) {
  std::string f(fn);
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, f + ": dtype of k_new/v_new");
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, f + ": head_dim must be 64 or 128");
  if (block_size != kBlock) return fail(PKV_ERR_UNSUPPORTED, f + ": block_size must be 16");
  if (batch < 0 || n_kv_heads < 1 || max_blocks_per_seq < 1 || num_pages < 1)
    return fail(PKV_ERR_INVALID_ARG, f + ": bad batch/n_kv_heads/max_blocks/num_pages");
  if (static_cast<int64_t>(batch) * n_kv_heads >= (int64_t{1} << 31) ||
      static_cast<int64_t>(batch) * max_blocks_per_seq >= (int64_t{1} << 31))
    return fail(PKV_ERR_UNSUPPORTED, f + ": batch too large");
  if (batch == 0) return ok();
  if (!k_new || !v_new || !k_codes || !v_codes || !meta || !block_table || !positions || !aligned(k_new, 4) ||
      !aligned(v_new, 4) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(meta, 16) ||
      !aligned(block_table, 4) || !aligned(positions, 4))
    return fail(PKV_ERR_INVALID_ARG, f + ": NULL or misaligned pointer");
  const int grid = (batch * n_kv_heads + kWavesPerGroup - 1) / kWavesPerGroup;
  auto kern = dtype == PKV_BF16 ? append_q8_kernel<true> : append_q8_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kWave * kWavesPerGroup), 0, static_cast<hipStream_t>(stream), k_new,
                     v_new, static_cast<uint8_t*>(k_codes), static_cast<uint8_t*>(v_codes),
                     static_cast<float*>(meta), block_table, positions, from_lens ? 1 : 0, batch, n_kv_heads,
                     head_dim, max_blocks_per_seq, num_pages);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail((f + " launch").c_str(), e);
  return ok();
}

}  // namespace
}  // namespace pkv

using pkv::fail;
using pkv::ok;

extern "C" {

int pkv_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                  const int32_t* block_table, const int32_t* positions, int32_t batch,
                  int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t max_blocks_per_seq, int32_t num_pages, int32_t dtype, void* stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "pkv_kv_append: dtype");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_kv_append: head_dim must be 64 or 128");
  if (block_size != pkv::kBlock) return fail(PKV_ERR_UNSUPPORTED, "pkv_kv_append: block_size must be 16");
  if (batch < 0 || n_kv_heads < 1 || max_blocks_per_seq < 1 || num_pages < 1)
    return fail(PKV_ERR_INVALID_ARG, "pkv_kv_append: bad batch/n_kv_heads/max_blocks/num_pages");
  if (static_cast<int64_t>(batch) * n_kv_heads >= (int64_t{1} << 31) ||
      static_cast<int64_t>(batch) * max_blocks_per_seq >= (int64_t{1} << 31))
    return fail(PKV_ERR_UNSUPPORTED, "pkv_kv_append: batch too large");
  if (batch == 0) return ok();
  if (!k_new || !v_new || !k_pages || !v_pages || !block_table || !positions ||
      !pkv::aligned(k_new, 16) || !pkv::aligned(v_new, 4) || !pkv::aligned(k_pages, 16) ||
      !pkv::aligned(v_pages, 4) || !pkv::aligned(block_table, 4) || !pkv::aligned(positions, 4))
    return fail(PKV_ERR_INVALID_ARG, "pkv_kv_append: NULL or misaligned pointer");
  const int pairs = batch * n_kv_heads;
  const int grid = (pairs + pkv::kWavesPerGroup - 1) / pkv::kWavesPerGroup;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PKV_BF16)
    hipLaunchKernelGGL(pkv::append_kernel<2>, dim3(grid), dim3(256), 0, s, k_new, v_new, k_pages,
                       v_pages, block_table, positions, batch, n_kv_heads, head_dim,
                       max_blocks_per_seq, num_pages);
  else
    hipLaunchKernelGGL(pkv::append_kernel<4>, dim3(grid), dim3(256), 0, s, k_new, v_new, k_pages,
                       v_pages, block_table, positions, batch, n_kv_heads, head_dim,
                       max_blocks_per_seq, num_pages);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::hip_fail("append kernel launch", e);
  return ok();
}

int pkv_paged_decode_attn(const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, const int32_t* seq_lens, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                          void* out, void* stream, int32_t batch, int32_t max_blocks_per_seq,
                          int32_t num_pages, int32_t dtype, void* workspace,
                          size_t workspace_bytes, const pkv_decode_opts* opts) {
  return pkv::decode_common(true, true, "pkv_paged_decode_attn", q, nullptr, nullptr, k_pages, v_pages,
                            nullptr, block_table,
                            seq_lens, n_q_heads, n_kv_heads, head_dim, block_size, scale, out,
                            stream, batch, max_blocks_per_seq, num_pages, dtype, workspace,
                            workspace_bytes, opts);
}

int pkv_paged_decode_split(const void* q, const void* k_pages, const void* v_pages,
                           const int32_t* block_table, const int32_t* seq_lens, int32_t n_q_heads,
                           int32_t n_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                           void* out, void* stream, int32_t batch, int32_t max_blocks_per_seq,
                           int32_t num_pages, int32_t dtype, void* workspace,
                           size_t workspace_bytes, const pkv_decode_opts* opts) {
  return pkv::decode_common(true, false, "pkv_paged_decode_split", q, nullptr, nullptr, k_pages,
                            v_pages, nullptr, block_table, seq_lens, n_q_heads, n_kv_heads, head_dim, block_size,
                            scale, out, stream, batch, max_blocks_per_seq, num_pages, dtype,
                            workspace, workspace_bytes, opts);
}

int pkv_decode_step(const void* q, const void* k_new, const void* v_new, void* k_pages,
                    void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                    float scale, void* out, void* stream, int32_t batch,
                    int32_t max_blocks_per_seq, int32_t num_pages, int32_t dtype, void* workspace,
                    size_t workspace_bytes, const pkv_decode_opts* opts) {
  if (batch > 0 && (!k_new || !v_new))
    return fail(PKV_ERR_INVALID_ARG, "pkv_decode_step: k_new and v_new are required");
  return pkv::decode_common(true, true, "pkv_decode_step", q, k_new, v_new, k_pages, v_pages,
                            nullptr, block_table, seq_lens, n_q_heads, n_kv_heads, head_dim, block_size,
                            scale, out, stream, batch, max_blocks_per_seq, num_pages, dtype,
                            workspace, workspace_bytes, opts);
}

int pkv_decode_step_split(const void* q, const void* k_new, const void* v_new, void* k_pages,
                          void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                          int32_t block_size, float scale, void* out, void* stream, int32_t batch,
                          int32_t max_blocks_per_seq, int32_t num_pages, int32_t dtype,
                          void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts) {
  if (batch > 0 && (!k_new || !v_new))
    return fail(PKV_ERR_INVALID_ARG, "pkv_decode_step_split: k_new and v_new are required");
  return pkv::decode_common(true, false, "pkv_decode_step_split", q, k_new, v_new, k_pages,
                            v_pages, nullptr, block_table, seq_lens, n_q_heads, n_kv_heads, head_dim,
                            block_size, scale, out, stream, batch, max_blocks_per_seq, num_pages,
                            dtype, workspace, workspace_bytes, opts);
}

int pkv_decode_step_noalloc(const void* q, const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                            const int32_t* block_table, const int32_t* seq_lens, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, int32_t block_size, float scale, void* out,
                            void* stream, int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                            int32_t dtype, const pkv_decode_opts* opts) {
  if (batch > 0 && (!k_new || !v_new))
    return fail(PKV_ERR_INVALID_ARG, "pkv_decode_step_noalloc: k_new and v_new are required");
  return pkv::decode_common(true, true, "pkv_decode_step_noalloc", q, k_new, v_new, k_pages, v_pages, nullptr,
                            block_table, seq_lens, n_q_heads, n_kv_heads, head_dim, block_size, scale, out, stream,
                            batch, max_blocks_per_seq, num_pages, dtype, nullptr, 0, opts, 1, 0, true);
}

int pkv_lse_combine(const void* workspace, size_t workspace_bytes, const int32_t* seq_lens,
                    int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_blocks_per_seq, void* out, int32_t dtype,
                    const pkv_decode_opts* opts, void* stream) {
  return pkv::decode_common(false, true, "pkv_lse_combine", nullptr, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr,
                            seq_lens, n_q_heads, n_kv_heads, head_dim, block_size, 1.0f, out,
                            stream, batch, max_blocks_per_seq, 1, dtype,
                            const_cast<void*>(workspace), workspace_bytes, opts);
}

int pkv_paged_decode_multi(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t q_len, int32_t window, float scale, void* out,
                           void* stream, int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                           int32_t dtype, void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts) {
  return pkv::decode_common(true, true, "pkv_paged_decode_multi", q, nullptr, nullptr, k_pages, v_pages, nullptr,
                            block_table, seq_lens, n_q_heads, n_kv_heads, head_dim, block_size, scale, out, stream,
                            batch, max_blocks_per_seq, num_pages, dtype, workspace, workspace_bytes, opts, q_len,
                            window);
}

int pkv_paged_decode_attn_q8(const void* q, const void* k_codes, const void* v_codes, const void* meta,
                             const int32_t* block_table, const int32_t* seq_lens, int32_t n_q_heads,
                             int32_t n_kv_heads, int32_t head_dim, int32_t block_size, float scale, void* out,
                             void* stream, int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                             void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts) {
  return pkv::decode_common(true, true, "pkv_paged_decode_attn_q8", q, nullptr, nullptr, k_codes, v_codes,
                            meta, block_table, seq_lens, n_q_heads, n_kv_heads, head_dim, block_size, scale,
                            out, stream, batch, max_blocks_per_seq, num_pages, PKV_U8, workspace,
                            workspace_bytes, opts);
}

int pkv_paged_decode_split_q8(const void* q, const void* k_codes, const void* v_codes, const void* meta,
                              const int32_t* block_table, const int32_t* seq_lens, int32_t n_q_heads,
                              int32_t n_kv_heads, int32_t head_dim, int32_t block_size, float scale, void* out,
                              void* stream, int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                              void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts) {
  return pkv::decode_common(true, false, "pkv_paged_decode_split_q8", q, nullptr, nullptr, k_codes, v_codes,
                            meta, block_table, seq_lens, n_q_heads, n_kv_heads, head_dim, block_size, scale,
                            out, stream, batch, max_blocks_per_seq, num_pages, PKV_U8, workspace,
                            workspace_bytes, opts);
}

int pkv_decode_step_q8(const void* q, const void* k_new, const void* v_new, void* k_codes, void* v_codes,
                       void* meta, const int32_t* block_table, const int32_t* seq_lens, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, int32_t block_size, float scale, void* out,
                       void* stream, int32_t batch, int32_t max_blocks_per_seq, int32_t num_pages,
                       void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts) {
  if (batch > 0 && (!k_new || !v_new))
    return fail(PKV_ERR_INVALID_ARG, "pkv_decode_step_q8: k_new and v_new are required");
  return pkv::decode_common(true, true, "pkv_decode_step_q8", q, k_new, v_new, k_codes, v_codes, meta,
                            block_table, seq_lens, n_q_heads, n_kv_heads, head_dim, block_size, scale, out,
                            stream, batch, max_blocks_per_seq, num_pages, PKV_U8, workspace, workspace_bytes,
                            opts);
}

int pkv_kv_append_q8(const void* k_new, const void* v_new, void* k_codes, void* v_codes, void* meta,
                     const int32_t* block_table, const int32_t* positions, int32_t batch, int32_t n_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_pages,
                     int32_t dtype, void* stream) {
  return pkv::append_q8_common("pkv_kv_append_q8", k_new, v_new, k_codes, v_codes, meta, block_table, positions,
                               false, batch, n_kv_heads, head_dim, block_size, max_blocks_per_seq, num_pages,
                               dtype, stream);
}

int pkv_decode_resolve(int32_t dtype, int32_t head_dim, int32_t n_q_heads, int32_t n_kv_heads,
                       int32_t batch, int32_t max_blocks_per_seq, const pkv_decode_opts* opts,
                       pkv_decode_opts* resolved, int64_t* workspace_bytes) {
  if (!resolved || !workspace_bytes)
    return fail(PKV_ERR_INVALID_ARG, "pkv_decode_resolve: NULL output");
  int st = pkv::check_decode_shapes("pkv_decode_resolve", n_q_heads, n_kv_heads, head_dim, 16, batch,
                                    max_blocks_per_seq, 1, dtype);
  if (st != PKV_OK) return st;
  pkv::Resolved r;
  st = pkv::resolve_opts(dtype, head_dim, n_q_heads / n_kv_heads, batch, max_blocks_per_seq,
                         n_kv_heads, opts, &r);
  if (st != PKV_OK) return st;
  resolved->n_items = r.n_items;
  resolved->min_chunk_pages = r.min_chunk;
  resolved->combine_mode = r.combine_mode;
  resolved->schedule = r.schedule;
  *workspace_bytes = pkv_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, r.n_items);
  return *workspace_bytes < 0 ? static_cast<int>(*workspace_bytes) : ok();
}

int pkv_copy_blocks(void* k_pages, void* v_pages, const int32_t* src_pages,
                    const int32_t* dst_pages, int32_t n_pairs, int32_t n_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t num_pages, int32_t dtype,
                    void* stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "pkv_copy_blocks: dtype");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_copy_blocks: head_dim must be 64 or 128");
  if (block_size != pkv::kBlock) return fail(PKV_ERR_UNSUPPORTED, "pkv_copy_blocks: block_size must be 16");
  if (n_pairs < 0 || n_kv_heads < 1 || num_pages < 1 ||
      static_cast<int64_t>(n_pairs) * n_kv_heads >= (int64_t{1} << 31))
    return fail(PKV_ERR_INVALID_ARG, "pkv_copy_blocks: bad n_pairs/n_kv_heads/num_pages");
  if (n_pairs == 0) return ok();
  if (!k_pages || !v_pages || !src_pages || !dst_pages || !pkv::aligned(k_pages, 16) ||
      !pkv::aligned(v_pages, 16) || !pkv::aligned(src_pages, 4) || !pkv::aligned(dst_pages, 4))
    return fail(PKV_ERR_INVALID_ARG, "pkv_copy_blocks: NULL or misaligned pointer");
  const int tile = pkv::kBlock * head_dim * (dtype == PKV_BF16 ? 2 : 4);
  const int items = n_pairs * n_kv_heads;
  hipLaunchKernelGGL(pkv::copy_blocks_kernel, dim3((items + pkv::kWavesPerGroup - 1) / pkv::kWavesPerGroup),
                     dim3(256), 0, static_cast<hipStream_t>(stream), static_cast<char*>(k_pages),
                     static_cast<char*>(v_pages), src_pages, dst_pages, n_pairs, n_kv_heads, tile, num_pages);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::hip_fail("copy_blocks launch", e);
  return ok();
}

int pkv_gather_probe(const void* k_pages, const void* v_pages, const int32_t* block_table,
                     const int32_t* seq_lens, int32_t n_kv_heads, int32_t head_dim, int32_t batch,
                     int32_t max_blocks_per_seq, int32_t num_pages, int32_t dtype, int64_t page_stride_bytes,
                     int64_t head_stride_bytes, int32_t n_items, int32_t min_chunk_pages, void* sink,
                     size_t sink_bytes, void* stream) {
  int st = pkv::check_decode_shapes("pkv_gather_probe", n_kv_heads, n_kv_heads, head_dim, pkv::kBlock, batch,
                                    max_blocks_per_seq, num_pages, dtype);
  if (st != PKV_OK) return st;
  if (dtype == PKV_U8) return fail(PKV_ERR_UNSUPPORTED, "pkv_gather_probe: dense caches only (PKV_F32, PKV_BF16)");
  const int64_t tile = static_cast<int64_t>(pkv::kBlock) * head_dim * (dtype == PKV_BF16 ? 2 : 4);
  const int64_t hstride = head_stride_bytes > 0 ? head_stride_bytes : tile;
  const int64_t stride = page_stride_bytes > 0 ? page_stride_bytes : hstride * n_kv_heads;
  if (hstride < tile || hstride % 16 != 0 || stride < hstride * n_kv_heads || stride % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_gather_probe: head_stride_bytes must be 0 or a multiple of 16 of at "
                                     "least one tile, page_stride_bytes 0 or a multiple of 16 of at least "
                                     "n_kv_heads head strides");
  if (batch == 0) return ok();
  if (!k_pages || !v_pages || !block_table || !seq_lens || !sink || !pkv::aligned(k_pages, 16) ||
      !pkv::aligned(v_pages, 16) || !pkv::aligned(block_table, 4) || !pkv::aligned(seq_lens, 4) ||
      !pkv::aligned(sink, 4))
    return fail(PKV_ERR_INVALID_ARG, "pkv_gather_probe: NULL or misaligned pointer");
  pkv_decode_opts o{n_items, min_chunk_pages, 0, PKV_SCHEDULE_STATIC};
  pkv::Resolved r;
  st = pkv::resolve_opts(dtype, head_dim, 1, batch, max_blocks_per_seq, n_kv_heads, &o, &r);
  if (st != PKV_OK) return st;
  if (sink_bytes < static_cast<size_t>(r.n_items) * 4)
    return fail(PKV_ERR_INVALID_ARG, "pkv_gather_probe: sink needs 4 * n_items bytes (" +
                                         std::to_string(r.n_items) + " items)");
  pkv::DecodeArgs a{};
  a.k_pages = const_cast<void*>(k_pages);
  a.v_pages = const_cast<void*>(v_pages);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.n_q = n_kv_heads;
  a.n_kv = n_kv_heads;
  a.group = 1;
  a.q_len = 1;
  a.cols = 1;
  a.max_blocks = max_blocks_per_seq;
  a.num_pages = num_pages;
  a.n_items = r.n_items;
  a.min_chunk = r.min_chunk;
  const size_t lds = pkv::split_lds_bytes(batch);
  if (lds > pkv::kMaxLdsBytes) return fail(PKV_ERR_UNSUPPORTED, "pkv_gather_probe: batch too large");
  using Fn = void (*)(pkv::DecodeArgs, size_t, size_t, uint32_t*);
  const Fn fn = dtype == PKV_BF16
                    ? (head_dim == 128 ? pkv::gather_probe_kernel<true, 128, pkv::kPrefetchPages>
                                       : pkv::gather_probe_kernel<true, 64, pkv::kPrefetchPages>)
                    : (head_dim == 128 ? pkv::gather_probe_kernel<false, 128, 1>
                                       : pkv::gather_probe_kernel<false, 64, 1>);
  const int grid = (r.n_items + pkv::kWavesPerGroup - 1) / pkv::kWavesPerGroup;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(pkv::kWave * pkv::kWavesPerGroup), lds, static_cast<hipStream_t>(stream),
                     a, static_cast<size_t>(stride), static_cast<size_t>(hstride), static_cast<uint32_t*>(sink));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::hip_fail("gather probe launch", e);
  return ok();
}

int pkv_gather_probe_q8(const void* k_codes, const void* v_codes, const void* meta, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t n_kv_heads, int32_t head_dim, int32_t batch,
                        int32_t max_blocks_per_seq, int32_t num_pages, int32_t n_items, int32_t min_chunk_pages,
                        void* sink, size_t sink_bytes, void* stream) {
  int st = pkv::check_decode_shapes("pkv_gather_probe_q8", n_kv_heads, n_kv_heads, head_dim, pkv::kBlock, batch,
                                    max_blocks_per_seq, num_pages, PKV_U8);
  if (st != PKV_OK) return st;
  if (batch == 0) return ok();
  if (!k_codes || !v_codes || !meta || !block_table || !seq_lens || !sink || !pkv::aligned(k_codes, 16) ||
      !pkv::aligned(v_codes, 16) || !pkv::aligned(meta, 16) || !pkv::aligned(block_table, 4) ||
      !pkv::aligned(seq_lens, 4) || !pkv::aligned(sink, 4))
    return fail(PKV_ERR_INVALID_ARG, "pkv_gather_probe_q8: NULL or misaligned pointer");
  pkv_decode_opts o{n_items, min_chunk_pages, 0, PKV_SCHEDULE_STATIC};
  pkv::Resolved r;
  st = pkv::resolve_opts(PKV_U8, head_dim, 1, batch, max_blocks_per_seq, n_kv_heads, &o, &r);
  if (st != PKV_OK) return st;
  if (sink_bytes < static_cast<size_t>(r.n_items) * 4)
    return fail(PKV_ERR_INVALID_ARG, "pkv_gather_probe_q8: sink needs 4 * n_items bytes (" +
                                         std::to_string(r.n_items) + " items)");
  pkv::DecodeArgs a{};
  a.k_pages = const_cast<void*>(k_codes);
  a.v_pages = const_cast<void*>(v_codes);
  a.meta = meta;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.n_q = n_kv_heads;
  a.n_kv = n_kv_heads;
  a.group = 1;
  a.q_len = 1;
  a.cols = 1;
  a.max_blocks = max_blocks_per_seq;
  a.num_pages = num_pages;
  a.n_items = r.n_items;
  a.min_chunk = r.min_chunk;
  const size_t lds = pkv::split_lds_bytes(batch);
  if (lds > pkv::kMaxLdsBytes) return fail(PKV_ERR_UNSUPPORTED, "pkv_gather_probe_q8: batch too large");
  using Fn = void (*)(pkv::DecodeArgs, uint32_t*);
  const Fn fn = head_dim == 128 ? pkv::gather_probe_q8_kernel<128, PKV_Q8_PREFETCH_PAGES>
                                : pkv::gather_probe_q8_kernel<64, PKV_Q8_PREFETCH_PAGES>;
  const int grid = (r.n_items + pkv::kWavesPerGroup - 1) / pkv::kWavesPerGroup;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(pkv::kWave * pkv::kWavesPerGroup), lds, static_cast<hipStream_t>(stream),
                     a, static_cast<uint32_t*>(sink));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::hip_fail("gather probe launch", e);
  return ok();
}

int pkv_hbm_read_probe(const void* buf, size_t bytes, void* sink, int32_t n_blocks, void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || !pkv::aligned(buf, 16) || !pkv::aligned(sink, 4) ||
      n_blocks < 1)
    return fail(PKV_ERR_INVALID_ARG, "pkv_hbm_read_probe: bad argument");
  hipLaunchKernelGGL(pkv::read_probe_kernel, dim3(n_blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const pkv::u32x4*>(buf), bytes / 16,
                     static_cast<uint32_t*>(sink));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::hip_fail("read probe launch", e);
  return ok();
}

int pkv_launch_probe(int32_t mode, int32_t grid, int32_t iters, int32_t* bar, float* us_per_launch, void* stream) {
  if (mode < 0 || mode > 2 || grid < 0 || iters < 1 || us_per_launch == nullptr || (mode == 2 && bar == nullptr) ||
      (bar != nullptr && !pkv::aligned(bar, 4)))
    return fail(PKV_ERR_INVALID_ARG, "pkv_launch_probe: bad argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0, n_cu = 0, coop = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
  if (e != hipSuccess) return pkv::hip_fail("launch probe device query", e);
  if (mode > 0 && !coop) return fail(PKV_ERR_UNSUPPORTED, "pkv_launch_probe: no cooperative launch on this device");
  if (grid == 0) grid = n_cu;
  int* bar_arg = bar;
  int barrier = mode == 2 ? 1 : 0;
  int spin_limit = 1 << 20;
  void* args[] = {&bar_arg, &barrier, &spin_limit};
  auto launch = [&]() -> hipError_t {
    if (mode == 0) {
      hipLaunchKernelGGL(pkv::launch_probe_kernel, dim3(grid), dim3(256), 0, s, bar_arg, barrier, spin_limit);
      return hipGetLastError();
    }
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(pkv::launch_probe_kernel), dim3(grid), dim3(256),
                                      args, 0, s);
  };
  hipEvent_t e0 = nullptr, e1 = nullptr;
  e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  for (int i = 0; i < 5 && e == hipSuccess; ++i) e = launch();   // warm-up
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  for (int i = 0; i < iters && e == hipSuccess; ++i) e = launch();
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return pkv::hip_fail("launch probe", e);
  *us_per_launch = 1000.f * ms / static_cast<float>(iters);
  return ok();
}

int pkv_copy_probe(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes % 16 != 0 || !pkv::aligned(dst, 16) || !pkv::aligned(src, 16))
    return fail(PKV_ERR_INVALID_ARG, "pkv_copy_probe: bad argument");
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return pkv::hip_fail("copy probe device query", e);
  hipLaunchKernelGGL(pkv::copy_probe_kernel, dim3(n_cu * 8), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<pkv::u32x4*>(dst),
                     static_cast<const pkv::u32x4*>(src), bytes / 16);
  e = hipGetLastError();
  if (e != hipSuccess) return pkv::hip_fail("copy probe launch", e);
  return ok();
}

}  // extern "C"
