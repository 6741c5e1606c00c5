// DeFT tree attention on gfx950: partial-attention kernels and the
// log-sum-exp merge kernel, plus the C-ABI entry points that launch them.
//
// Sources (the DeFT pages: arXiv 2404.00242, abstract; "DeFT Guide: Flash
// Tree-Attention for LLM Serving"):
//   - "Tree-Constrained Attention Formulation": a query attends, with scale
//     1/sqrt(d), to the tokens of its node and of every ancestor;
//   - "1. KV-Guided Grouping": a chunk of KV is read from HBM once for all
//     queries that need it; here one work-group streams one chunk for one KV
//     head and scores every grouped query and every query head sharing that
//     KV head (grouped-query attention), the tree bitmask selecting the
//     visible tokens;
//   - "2. Flattened Tree KV Splitting": the work unit is an equal-sized chunk
//     of the flattened tree KV;
//   - "The Online Softmax Tile Accumulation": running max, running sum and a
//     rescaled output accumulator per row; per-chunk results (O, m, l) are
//     merged by the same rule in a second kernel;
//   - "Integration with Paged KV Caches" / "2. Paged KV-Cache Compatibility":
//     a chunk's flat tokens are mapped to pool rows through the block table
//     once per work-group, outside the inner loops.
//
// Row convention: for KV head g and chunk c with group slots j = 0..n-1, row
// r = j * G + hh is slot j's query on query head g * G + hh (G = Hq / Hkv).
//
// One partial kernel (partial_attention) runs two bodies on one work description:
//   mfma_body  bf16 chunks (rows padded up to the 16-row MFMA tile):
//              16x16x32 bf16 MFMA for S = K Q^T and O^T = V^T P^T, 64 rows
//              per work-group, the chunk's tokens split across 4 wave pairs
//              and the splits merged in LDS (or 128 rows, 2 splits of 4
//              waves, for wide items);
//   valu_body  fp32 inputs, and bf16 chunks below the DEFT_MFMA_MIN_ROWS
//              threshold when one is set (default 1: none): per-token dot
//              products with wavefront reductions.
// Scores are kept in log2 units (scale * log2(e) folded in) so exp2 is used;
// the stored m is converted back to natural-log units.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <string>
#include <cstdint>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "deft_internal.h"

namespace deft {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -INFINITY;
// A running max is only raised once a row's max exceeds it by this many
// log2 units; the probabilities then stay below 2^8 and the accumulators
// are rescaled rarely.  The stored partial is renormalised to the true max.
constexpr float kRescaleSlack = 8.0f;

struct DevPlan {
  const int32_t* chunk_start;
  const int32_t* group_offsets;
  const int32_t* chunk_full;
  const int32_t* slot_query;
  const uint32_t* slot_mask;
  const int32_t* flat_to_logical;
  const int32_t* query_slot_offsets;
  const int32_t* query_slots;
  const int4* mfma_items;
  const int4* valu_items;
  int32_t* tickets;          // [Nq * Hq], zero between calls (fused merge)
  int32_t* status;           // 1 once a bounded wait gave up (deft_plan_status reads and clears it)
  const int32_t* merge_slots;   // [Nq][merge_stride] slot ids padded with -1, or unused
  int32_t n_mfma_group, n_mfma_wide, n_mfma, n_valu, mask_words, num_queries, merge_stride;   // mfma_items: group, wide, 64-row
};

// Operands of the per-(query, head) merge (the merge kernel and the fused
// tail of the partial kernels).
struct MergeArgs {
  const float* po;
  const float* pm;
  const float* pl;
  void* out;
  const int32_t* query_slot_offsets;
  const int32_t* query_slots;
  const int32_t* merge_slots;   // fixed-stride lists (merge_stride > 0) or unused
  int32_t nq, hq, po_bf16, merge_stride;
};

struct PartialArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  float* po;         // partial O: fp32 unnormalised, or bf16 divided by l (po_bf16)
  float* pm;
  float* pl;
  DevPlan plan;
  int32_t hq, hkv, grp;
  int32_t po_bf16;   // 1: store O / l rounded to bf16 (internal workspace format)
  float scale_log2;  // log2(e) / sqrt(d)
  int32_t spin_limit;   // checks of a bounded inter-wave wait before it gives up
  int32_t fused;     // 1: single-dispatch launch (fused_publish, merge_worker)
  int32_t merge_wg_rows;   // (query, head) rows per merge work-group when fused
  int32_t max_valu_rows;   // host only: picks the VALU kernel's row capacity
  MergeArgs merge;   // used when fused
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over aligned groups of N lanes (N = 4, 8, 16 or 32), every lane of a
// group receiving the group's sum, with DPP lane moves on the VALU (no LDS
// crossbar): swaps within quads, then mirrors within half-rows and rows of
// 16 lanes (after the previous steps every lane of a subgroup holds the same
// partial sum, so a mirror pairs each subgroup with its neighbour), then a
// swap of adjacent 16-lane rows.
template <int N>
__device__ inline float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
  x += dpp(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
  if constexpr (N >= 16) x += dpp(x, std::integral_constant<int, 0x140>{});  // row_mirror
  if constexpr (N >= 32) {
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
  return x;
}

// s + the dot product of 8 packed bf16 pairs (four words each), fp32
// accumulate.  Written as inline asm: built from register words through the
// fdot2 builtin and bit casts, the compiler fed one register to every call
// of an unrolled sequence.  The compiler cannot see the asm's VGPR write, so
// the asm itself provides the two wait states a following DPP read of the
// result needs.
__device__ inline float dot8_bf16(const u32x4& a, const uint32_t* b, float s) {
  asm("v_dot2c_f32_bf16 %0, %1, %2\n\t"
      "v_dot2c_f32_bf16 %0, %3, %4\n\t"
      "v_dot2c_f32_bf16 %0, %5, %6\n\t"
      "v_dot2c_f32_bf16 %0, %7, %8\n\t"
      "s_nop 1"
      : "+v"(s)
      : "v"(a[0]), "v"(b[0]), "v"(a[1]), "v"(b[1]), "v"(a[2]), "v"(b[2]), "v"(a[3]), "v"(b[3]));
  return s;
}

// Two floats rounded to bf16 (nearest even) by one v_cvt_pk_bf16_f32, lo in
// the low half.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static void unpack(const u32x4& r, float* out) {
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(r[i]);
  }
};

// Pool row (page * 16 + slot) of every flat token of the chunk, into LDS,
// stored as row * mul + add.  All flat-to-logical loads are issued before any
// block-table load so the two dependent lookups cost two memory latencies,
// not two per token; a chunk whose tokens are one run of consecutive logical
// tokens (lstart >= 0, its first token's logical index) needs no
// flat-to-logical lookup at all, only the block-table one.  mid() runs right
// after the block-table loads are issued (callers issue their own
// independent loads there, so those overlap the last lookup).  With RPI > 0 the rows of each 32-token step are stored
// permuted, entry (t % RPI) * (32 / RPI) + (t % 32) / RPI, which puts the rows
// one lane of a direct-to-LDS load sequence needs next to each other.  NT is
// the work-group size.
template <int RPI, int NT, int N, typename Mid>
__device__ inline void stage_token_rows_n(int32_t* tok_row, const DevPlan& P, const int32_t* bt,
                                          int32_t cs, int32_t len, int32_t lstart, int32_t mul, int32_t add,
                                          Mid mid) {
  // N fixed loads per thread and no branches: indices past the chunk end
  // re-read its last token, and their entries (t < N * NT <= kMaxChunkTokens)
  // are stored too, so every 32-token step up to N * NT has valid rows (the
  // MFMA body reads a partial last step whole; its extra tokens are masked).
  // A conditional store would also let the compiler sink the loads into it
  // and serialise them.
  int32_t lt[N];
  if (lstart >= 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) lt[k] = lstart + min(static_cast<int>(threadIdx.x) + k * NT, len - 1);
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k)
      lt[k] = P.flat_to_logical[cs + min(static_cast<int>(threadIdx.x) + k * NT, len - 1)];
  }
  int32_t pg[N];
#pragma unroll
  for (int k = 0; k < N; ++k) pg[k] = bt[lt[k] >> 4];
  mid();
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int t = threadIdx.x + k * NT;
    int at = t;
    if constexpr (RPI > 0) at = (t & ~31) + (t % RPI) * (32 / RPI) + (t & 31) / RPI;
    tok_row[at] = (pg[k] * kPageSize + (lt[k] & (kPageSize - 1))) * mul + add;
  }
}
template <int RPI, int NT, typename Mid>
__device__ inline void stage_token_rows(int32_t* tok_row, const DevPlan& P, const int32_t* bt,
                                        int32_t cs, int32_t len, int32_t lstart, int32_t mul, int32_t add,
                                        Mid mid) {
  static_assert(kMaxChunkTokens <= 16 * NT, "at most 16 staging batches");
  // N * NT stays within kMaxChunkTokens: N is the power of two at or above
  // ceil(len / NT) and NT divides kMaxChunkTokens.
  static_assert(kMaxChunkTokens % NT == 0, "whole staging batches");
  const int nk = (len + NT - 1) / NT;
  if (nk <= 1) stage_token_rows_n<RPI, NT, 1>(tok_row, P, bt, cs, len, lstart, mul, add, mid);
  else if (nk <= 2) stage_token_rows_n<RPI, NT, 2>(tok_row, P, bt, cs, len, lstart, mul, add, mid);
  else if (nk <= 4) stage_token_rows_n<RPI, NT, 4>(tok_row, P, bt, cs, len, lstart, mul, add, mid);
  else if (nk <= 8) stage_token_rows_n<RPI, NT, 8>(tok_row, P, bt, cs, len, lstart, mul, add, mid);
  else stage_token_rows_n<RPI, NT, 16>(tok_row, P, bt, cs, len, lstart, mul, add, mid);
}

// ---------------------------------------------------------------------------
// Merge kernel: four (query, query head) rows per wave, one per 16-lane row
// of lanes (merge_rows below).
// ---------------------------------------------------------------------------

// Whole-wave reductions without the LDS crossbar: DPP within each row of 16
// lanes, then the lane^16 and lane^32 exchanges by permlane swaps.
template <typename Op>
__device__ inline float wave_reduce(float x, Op op) {
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  x = op(x, dpp(x, std::integral_constant<int, 0xB1>{}));    // quad_perm [1,0,3,2]
  x = op(x, dpp(x, std::integral_constant<int, 0x4E>{}));    // quad_perm [2,3,0,1]
  x = op(x, dpp(x, std::integral_constant<int, 0x141>{}));   // row_half_mirror
  x = op(x, dpp(x, std::integral_constant<int, 0x140>{}));   // row_mirror
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(b[0]), __uint_as_float(b[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ inline float wave_max(float x) { return wave_reduce(x, [](float a, float b) { return fmaxf(a, b); }); }
__device__ inline float wave_sum(float x) { return wave_reduce(x, [](float a, float b) { return a + b; }); }
// Reduction over lanes l ^ k for k = LPT .. 32 (the lanes that hold the same
// position of different LPT-lane groups), in every lane: DPP row_ror:8 for
// the lane^8 exchange within a 16-lane row, then permlane swaps.
template <int LPT, typename Op>
__device__ inline float cross_group_reduce(float x, Op op) {
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "group width");
  if constexpr (LPT <= 8)
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)));
  if constexpr (LPT <= 16) {
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// Sum of lanes l, l^16, l^32, l^48 (the four 16-lane groups), in every lane.
__device__ inline float groups4_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Broadcast lane J of each 16-lane row to the whole row (DPP row_newbcast).
template <int J>
__device__ inline int row_bcast(int x) { return __builtin_amdgcn_update_dpp(0, x, 0x150 + J, 0xf, 0xf, false); }
template <int J>
__device__ inline float row_bcast(float x) { return __int_as_float(row_bcast<J>(__float_as_int(x))); }
// Max / sum over each 16-lane row (DPP), in every lane of the row.
template <typename Op>
__device__ inline float row_reduce16(float x, Op op) {
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  x = op(x, dpp(x, std::integral_constant<int, 0xB1>{}));    // quad_perm [1,0,3,2]
  x = op(x, dpp(x, std::integral_constant<int, 0x4E>{}));    // quad_perm [2,3,0,1]
  x = op(x, dpp(x, std::integral_constant<int, 0x141>{}));   // row_half_mirror
  return op(x, dpp(x, std::integral_constant<int, 0x140>{}));   // row_mirror
}

// Accesses of partial results.  COHERENT (the single-dispatch path, whose
// merge work-groups read partials that partial work-groups of the same
// launch wrote, possibly on other XCDs with their own L2): relaxed
// device-scope atomic stores and loads, which the compiler emits as ordinary
// vector memory instructions with device coherence scope (sc1 on gfx950:
// stores written through to the device's coherence point, loads served from
// it), so no write-back or invalidation of a whole L2 is needed to hand
// partials from one work-group to another; ordering comes from each wave's
// wait for its own stores and a work-group barrier before the relaxed
// ticket, and on the reading side from the ticket load the merge's loads
// depend on.  The two-dispatch path (kernel boundary in between) uses plain
// accesses.
template <bool COHERENT>
__device__ inline void st_u32(void* p, uint32_t v) {
  if constexpr (COHERENT) __hip_atomic_store(static_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *static_cast<uint32_t*>(p) = v;
}
template <bool COHERENT>
__device__ inline void st_f32(float* p, float v) { st_u32<COHERENT>(p, __float_as_uint(v)); }
template <bool COHERENT>
__device__ inline void st_u32x2(void* p, uint32_t lo, uint32_t hi) {
  if constexpr (COHERENT)
    __hip_atomic_store(static_cast<uint64_t*>(p), (static_cast<uint64_t>(hi) << 32) | lo, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else *static_cast<u32x2*>(p) = u32x2{lo, hi};
}
template <bool COHERENT>
__device__ inline void st_f32x4(float* p, f32x4 v) {
  if constexpr (COHERENT) {
    st_u32x2<true>(p, __float_as_uint(v[0]), __float_as_uint(v[1]));
    st_u32x2<true>(p + 2, __float_as_uint(v[2]), __float_as_uint(v[3]));
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}
template <bool COHERENT>
__device__ inline float ld_f32(const float* p) {
  if constexpr (COHERENT)
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
  else return *p;
}
template <bool COHERENT>
__device__ inline u32x2 ld_u32x2(const void* p) {
  if constexpr (COHERENT) {
    const uint64_t v = __hip_atomic_load(static_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return u32x2{static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32)};
  } else {
    return *static_cast<const u32x2*>(p);
  }
}
template <bool COHERENT>
__device__ inline u32x4 ld_u32x4(const void* p) {
  if constexpr (COHERENT) {
    const u32x2 a = ld_u32x2<true>(p), b = ld_u32x2<true>(static_cast<const char*>(p) + 8);
    return u32x4{a[0], a[1], b[0], b[1]};
  } else {
    return *static_cast<const u32x4*>(p);
  }
}

// Partial-result format of a merge: read from MergeArgs at run time, or
// fixed by a caller that knows it.
constexpr int kFmtRuntime = -1, kFmtF32 = 0, kFmtBf16 = 1;

// EPL consecutive elements of one partial O row (slot-head sh) as raw words:
// bf16 (O / l) or fp32 (unnormalised O).
template <int EPL, int FMT>
struct PartialRow {
  static constexpr int WORDS = FMT == kFmtBf16 ? EPL / 2 : EPL;
  uint32_t w[WORDS];
};
template <int FMT>
__device__ inline bool fmt_bf16(const MergeArgs& a) {
  if constexpr (FMT == kFmtRuntime) return a.po_bf16 != 0;
  else return FMT == kFmtBf16;
}
template <int D, int EPL, int FMT, bool COHERENT>
__device__ inline void load_partial_row(const MergeArgs& a, int64_t sh, int sub, PartialRow<EPL, FMT>& r) {
  if (fmt_bf16<FMT>(a)) {
    const uint16_t* src = reinterpret_cast<const uint16_t*>(a.po) + sh * D + sub * EPL;
    if constexpr (EPL == 8) {
      const u32x4 v = ld_u32x4<COHERENT>(src);
#pragma unroll
      for (int e = 0; e < 4; ++e) r.w[e] = v[e];
    } else {
      const u32x2 v = ld_u32x2<COHERENT>(src);
      r.w[0] = v[0];
      r.w[1] = v[1];
    }
    // with the format chosen at run time, every word is defined on both
    // branches, which keeps the row in registers
    if constexpr (FMT == kFmtRuntime) {
#pragma unroll
      for (int e = EPL / 2; e < EPL; ++e) r.w[e] = 0u;
    }
  } else if constexpr (FMT != kFmtBf16) {
    const float* src = a.po + sh * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const u32x4 v = ld_u32x4<COHERENT>(src + e);
#pragma unroll
      for (int k = 0; k < 4; ++k) r.w[e + k] = v[k];
    }
  }
}
template <int EPL, int FMT>
__device__ inline float partial_elem(const MergeArgs& a, const PartialRow<EPL, FMT>& r, int e) {
  if (fmt_bf16<FMT>(a)) return __uint_as_float(e & 1 ? (r.w[e >> 1] & 0xffff0000u) : (r.w[e >> 1] << 16));
  if constexpr (FMT != kFmtBf16) return __uint_as_float(r.w[e]);
  else return 0.f;
}
// Lane J's value of each 16-lane row, J = 0..15, in every lane of the row.
template <typename X, int... J>
__device__ inline void row_bcast_all(X x, X (&out)[16], std::integer_sequence<int, J...>) {
  ((out[J] = row_bcast<J>(x)), ...);
}

// Merge of (query, query head) rows, one per 16-lane row of lanes (four per
// wave); `code` = qi * Hq + h of this lane's row, or -1 for none.  Lane sub
// of a row reads the metadata (slot id, m, l) of the row's slots sub,
// sub + 16, ... and D/16 consecutive elements of every slot's partial O row.
// A round of up to 16 slots costs two rounds of dependent loads (the slot
// ids, then m, l and the O rows together).  With M = max_s m_s and
// w_s = exp(m_s - M):
//   fp32 unnormalised partials   out = sum_s w_s O_s / sum_s w_s l_s
//   bf16 partials holding O_s/l_s out = sum_s w_s l_s (O_s/l_s) / sum_s w_s l_s
// Rows with more than 16 slots take several rounds, rescaled online.
// PRE: the caller has already read the row's slot count (cnt0; 0 for no
// row) and this lane's first slot id (raw0: slot sub of the row's list, or
// -1), so the first round starts with the partials' own loads.
template <typename T, int D, bool COHERENT, int FMT, bool PRE = false>
__device__ __attribute__((always_inline)) void merge_rows(const MergeArgs& a, int code, int raw0 = -1,
                                                          int cnt0 = 0) {
  constexpr int EPL = D / 16;      // elements per lane
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const bool live = code >= 0;
  const int qi = live ? code / a.hq : 0, h = live ? code % a.hq : 0;
  // the row's slot list: fixed stride (padded with -1, read without a
  // dependent offset lookup) or CSR
  auto slot_list = [&](int& n) {
    if (a.merge_stride > 0) {
      n = a.merge_stride;
      return a.merge_slots + static_cast<size_t>(qi) * a.merge_stride;
    }
    const int s0 = a.query_slot_offsets[qi];
    n = a.query_slot_offsets[qi + 1] - s0;
    return a.query_slots + s0;
  };
  const int32_t* list = nullptr;   // with PRE, looked up only for rows of more than 16 slots
  int cnt;
  if constexpr (PRE) {
    cnt = live ? cnt0 : 0;
  } else {
    int n;
    list = slot_list(n);
    cnt = live ? n : 0;
  }
  const int cmax = static_cast<int>(wave_max(static_cast<float>(cnt)));
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float mrun = kNegInf, wsum = 0.f;
  for (int i0 = 0; i0 < cmax; i0 += 16) {
    int raw;
    if (PRE && i0 == 0) {
      raw = live ? raw0 : -1;
    } else {
      if (PRE && i0 == 16 && live) {
        int n;
        list = slot_list(n);
      }
      raw = i0 + sub < cnt ? list[i0 + sub] : -1;
    }
    // every slot's m, l and O row of this round, issued before any reduction
    const bool ok = raw >= 0;                   // padding entries are -1
    const int64_t sh = static_cast<int64_t>(ok ? raw : 0) * a.hq + h;
    const float mv = ok ? ld_f32<COHERENT>(a.pm + sh) : kNegInf;
    const float lv = ok ? ld_f32<COHERENT>(a.pl + sh) : 0.f;
    int sj[16];
    row_bcast_all(raw, sj, std::make_integer_sequence<int, 16>{});
    PartialRow<EPL, FMT> rows[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (sj[j] >= 0) load_partial_row<D, EPL, FMT, COHERENT>(a, static_cast<int64_t>(sj[j]) * a.hq + h, sub, rows[j]);
    const float mnew = fmaxf(mrun, row_reduce16(mv, [](float x, float y) { return fmaxf(x, y); }));
    const float w = mv == kNegInf ? 0.f : __expf(mv - mnew);
    const float wl = w * lv;
    const float wt = fmt_bf16<FMT>(a) ? wl : w;      // weight of the stored O row
    const float rescale = mrun == kNegInf ? 0.f : __expf(mrun - mnew);
    mrun = mnew;
    wsum = wsum * rescale + row_reduce16(wl, [](float x, float y) { return x + y; });
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= rescale;
    float wj[16];
    row_bcast_all(wt, wj, std::make_integer_sequence<int, 16>{});
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (sj[j] >= 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wj[j], partial_elem<EPL, FMT>(a, rows[j], e), acc[e]);
      }
  }
  if (!live) return;
  const float inv = 1.f / wsum;
  const size_t ob = (static_cast<size_t>(qi) * a.hq + h) * D + sub * EPL;
  if constexpr (sizeof(T) == 2) {
    uint32_t pk[EPL / 2];
#pragma unroll
    for (int e = 0; e < EPL / 2; ++e)
      pk[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    if constexpr (EPL == 8) *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + ob) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    else *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + ob) = u32x2{pk[0], pk[1]};
  } else {
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ob + e) =
          f32x4{acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void lse_merge(MergeArgs a) {
  const int wave0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4;
  if (wave0 >= a.nq * a.hq) return;          // whole waves leave together
  const int code = wave0 + ((threadIdx.x & 63) >> 4);
  merge_rows<T, D, false, kFmtRuntime>(a, code < a.nq * a.hq ? code : -1);
}

// ---------------------------------------------------------------------------
// Single-dispatch step.  The grid holds the partial work-groups followed by
// merge work-groups of 16 or 32 (query, query head) rows each.  A
// partial work-group stores its partials with device-coherent accesses
// (st_* with COHERENT), every wave waits for its own stores to complete, the
// work-group meets at a barrier, and it adds one to a ticket per (query,
// head) row it wrote (a relaxed device-scope atomic whose old value is not
// returned), then leaves.  A merge work-group reads its rows' slot counts
// and first slot ids, polls the rows' tickets until each has counted every
// slot of its query (a bounded wait: past the spin limit it reports a
// give-up through the plan's status word and merges what is there), takes
// that count back out of them (so that every ticket is zero again once the
// call has ended, give-up or not), and merges the rows through the same
// per-(query, head) merge as the merge kernel, with device-coherent loads.
//
// The dispatcher places work-groups in index order, so a merge work-group
// only takes a compute unit once every partial work-group has been placed,
// and no partial work-group waits for anything.  The merge reads spread over
// many work-groups (a merge by the work-group that completes a row would
// gather them on the few that finish last), and no
// write-back or invalidation of a whole L2 is needed (which would also throw
// other work-groups' KV out of their XCD's L2).  Calls that share a plan
// (and so its tickets) must not overlap.
// ---------------------------------------------------------------------------
// A bounded wait that ran out of checks: the work-group's results are
// invalid; the plan's status word (device memory) records it for
// deft_plan_status.
__device__ inline void report_give_up(int32_t* status, int lane) {
  if (lane == 0) __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int kPartialThreads = 512;    // threads of a partial-kernel work-group
// Rows per merge work-group: 16 (four waves of 4 rows) while that keeps the
// merge work-groups within kMergeWorkGroups, else 32 (eight waves), so that
// the merge reads spread over many compute units without the merge
// work-groups outnumbering them by far (measured on the 4K-prefix, parallel
// sampling, reasoning and multi-token trees: 8 rows, or 64 rows at two per
// lane row, were slower).
constexpr int kMergeWorkGroups = 128;
inline int merge_worker_rows(int nrows) { return (nrows + 15) / 16 <= kMergeWorkGroups ? 16 : 32; }

// End of a partial work-group on the single-dispatch path: tickets of rows
// [rb, rb + nr) of its item, once its partial stores have completed.
template <int ROWS>
__device__ __attribute__((always_inline)) void fused_publish(const DevPlan& P, int hq, int grp, int32_t rb,
                                                             int32_t nr, int32_t gofs, int g) {
  static_assert(ROWS <= kPartialThreads, "one ticket lane per row");
  const int r = static_cast<int>(threadIdx.x);
  int32_t* t = nullptr;
  if (r < nr) {      // the ticket's address is looked up while the stores drain
    const int row = rb + r;
    const int qi = P.slot_query[gofs + row / grp];
    t = P.tickets + static_cast<size_t>(qi) * hq + g * grp + row % grp;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (r < nr) __hip_atomic_fetch_add(t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge work-group mw of `rows` (query, head) rows (16 or 32): wave w
// merges rows mw * rows + 4 * w + (lane / 16).
template <typename T, int D>
__device__ __attribute__((always_inline)) void merge_worker(const MergeArgs& m, const DevPlan& P,
                                                            int32_t spin_limit, int mw, int rows) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, sub = lane & 15;
  const int nrows = m.nq * m.hq;
  const int code0 = mw * rows + w * 4;
  if (w * 4 >= rows || code0 >= nrows) return;     // whole waves leave together
  const int code = code0 + (lane >> 4);
  const bool live = code < nrows;
  const int qi = live ? code / m.hq : 0;
  // everything but the partials themselves, read before the wait
  const int need = live ? P.query_slot_offsets[qi + 1] - P.query_slot_offsets[qi] : 0;
  int n;
  const int32_t* list;
  if (m.merge_stride > 0) {
    n = m.merge_stride;
    list = m.merge_slots + static_cast<size_t>(qi) * m.merge_stride;
  } else {
    const int s0 = m.query_slot_offsets[qi];
    n = m.query_slot_offsets[qi + 1] - s0;
    list = m.query_slots + s0;
  }
  const int raw = live && sub < n ? list[sub] : -1;
  int32_t* t = P.tickets + (live ? code : 0);
  for (int spin = 0;; ++spin) {
    const int got = live ? __hip_atomic_load(t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : need;
    if (__all(got >= need)) break;
    if (spin >= spin_limit) {
      report_give_up(P.status, lane);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  // take this call's count back out rather than storing zero: after a
  // give-up, increments that arrive later still bring the ticket back to
  // zero by the end of the call
  if (live && sub == 0) __hip_atomic_fetch_add(t, -need, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the partials of this path: bf16 (O / l) for bf16 attention unless the
  // descriptor asks for fp32 ones, fp32 for fp32 (one format per launch, so
  // the branch is uniform)
  if (sizeof(T) == 2 && m.po_bf16)
    merge_rows<T, D, true, kFmtBf16, true>(m, live ? code : -1, raw, live ? n : 0);
  else
    merge_rows<T, D, true, kFmtF32, true>(m, live ? code : -1, raw, live ? n : 0);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS loads and wave helpers shared by the partial kernels.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lptr_t;
// Direct-to-LDS loads, written as inline asm: lane i's bytes land at LDS
// address lds + size * i (M0 holds the wave-uniform LDS base).  The compiler
// sees no LDS write here, so it adds no waits of its own for them; callers
// order them with explicit s_waitcnt vmcnt (they count as vector-memory loads).
// Work-group barrier for LDS data only: the wave's LDS operations complete,
// then s_barrier.  Unlike __syncthreads() it does not wait for the wave's
// outstanding global loads and stores, so loads issued before it (Q rows,
// the first step's K/V) stay in flight across it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lptr_t)p));
}
// `lds` is wave-uniform; readfirstlane only tells the compiler so (it keeps
// it in an SGPR at no cost where it can already prove it).
__device__ inline void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ inline void lds_dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory
// operations are outstanding / until all LDS operations are done.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 0xc07f;

// max over the 4 lanes that hold the same row (lanes l, l^16, l^32, l^48)
__device__ inline float rowmax4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float rowsum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two-wave rendezvous through LDS: publish `i` in *mine, then wait until
// *theirs reaches `i`.  Both waves of a pair run the same iteration count,
// so every wait ends; the spin is also bounded (`spins` checks, the kernel
// argument spin_limit) so that a broken pairing can never leave a wave that
// does not finish.  A wait that runs out of checks sets *status (device
// memory of the plan image) to 1: the work-group's results are then invalid,
// and deft_plan_status reports it to the host.  The flags are addressed as
// LDS (address space 3), so the accesses are ds_write / ds_read; through a
// generic pointer they would be flat accesses with device-coherence bits,
// which take the vector-memory path and cost several times the latency.
typedef __attribute__((address_space(3))) int32_t lds_i32;
__device__ inline lds_i32* as_lds(int32_t* p) { return (lds_i32*)p; }
__device__ inline void pair_sync(int32_t* mine, int32_t* theirs, int32_t i, int lane, int32_t spins,
                                 int32_t* status) {
  if (lane == 0) __hip_atomic_store(as_lds(mine), i, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  for (int spin = 0;; ++spin) {
    if (__hip_atomic_load(as_lds(theirs), __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= i) return;
    if (spin >= spins) break;
    __builtin_amdgcn_s_sleep(1);
  }
  report_give_up(status, lane);
}
// The same for N waves: wave `me` publishes `i` in flags[me], then waits
// until every other flag reaches `i` (bounded and reported like pair_sync).
template <int N>
__device__ inline void group_sync(int32_t* flags, int me, int32_t i, int lane, int32_t spins, int32_t* status) {
  if constexpr (N == 2) {
    pair_sync(&flags[me], &flags[me ^ 1], i, lane, spins, status);
  } else {
    // four flags (16-byte aligned) are read with one LDS load per check, so a
    // check costs one LDS round trip rather than three in a row
    static_assert(N == 4, "pairs or quads of waves");
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const volatile i32x4 lds_i32x4;
    if (lane == 0) __hip_atomic_store(as_lds(&flags[me]), i, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int spin = 0;; ++spin) {
      const i32x4 f = *(lds_i32x4*)as_lds(flags);
      if (min(min(f[0], f[1]), min(f[2], f[3])) >= i) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        return;
      }
      if (spin >= spins) break;
      __builtin_amdgcn_s_sleep(1);
    }
    report_give_up(status, lane);
  }
}

// ---------------------------------------------------------------------------
// VALU partial kernel: fp32 inputs (and bf16 chunks the DEFT_MFMA_MIN_ROWS
// threshold sends here); up to R rows per work-group (R = 4 or 8, the
// smaller that holds the plan's largest VALU work item; larger groups are
// split into items of 8 rows that share the chunk's KV through L2).  Scores and the PV update are wavefront arithmetic:
// lanes are grouped LPT per token (each lane holds 16 or 32 bytes of the
// token's K and V row), dot products are summed across the group with DPP
// moves; with bf16 inputs a lane's two tokens of a step share one dot2 per
// O element.  The work is a stream over the chunk's KV rows with little
// arithmetic per byte, so memory is fed like the MFMA kernel: each of the NW
// waves takes the chunk's steps (4 KB of K rows per step) w, w+NW, ... and
// streams them with direct-to-LDS loads into a private NSTG-stage ring,
// NSTG-1 steps ahead, with explicit waits.  Each lane group keeps its own
// online-softmax state (running max raised lazily); groups and waves are
// merged at the end.
// ---------------------------------------------------------------------------
template <int R> constexpr int valu_waves() { return R <= 8 ? 8 : 4; }

template <typename T, int D, int R>
struct ValuShape {
  static constexpr int EB = sizeof(T);
  static constexpr int NW = valu_waves<R>();
  static constexpr int TILE_B = 4096;
  static constexpr int NSTG = NW == 8 ? 2 : 4;
  static constexpr int STAGE_B = 2 * TILE_B + 256;
  static constexpr int RING_B = NW * NSTG * STAGE_B;
  static constexpr int RED_B = NW * R * (D + 2) * 4;
  static constexpr int SMEM_B = RING_B > RED_B ? RING_B : RED_B;
  // LDS carve-out: ring / reduction buffer, staged token rows, fused-merge lists
  static constexpr int TOK_OFF = SMEM_B;
  static constexpr int LDS_B = TOK_OFF + 4 * kMaxChunkTokens;
};

template <typename T, int D, int R, bool FUSED>
__device__ __forceinline__ void valu_body(const PartialArgs& a, char* lds, int bid) {
  constexpr int EB = sizeof(T);
  // bytes of each K and V row a lane holds: 32 for bf16 d=128 with up to 4
  // rows (8 lanes per token: the per-token softmax work is shared by fewer
  // lanes), else 16 (the rows' accumulators would not fit)
  constexpr int LB = (EB == 2 && D == 128 && R <= 4) ? 32 : 16;
  constexpr int NLD = LB / 16;                     // 16-byte reads per lane and row
  constexpr int EPL = LB / EB;                     // elements per lane
  constexpr int LPT = D / EPL;                     // lanes per token
  constexpr int TPW = 64 / LPT;                    // tokens per wave pass
  // two waves per SIMD (latency hiding) while the rows' registers allow it
  constexpr int NW = valu_waves<R>();
  constexpr int ROWB = D * EB;                     // bytes per token row
  constexpr int CH = ROWB / 16;                    // 16-byte chunks per row
  constexpr int TILE_B = 4096;                     // K (or V) bytes per step
  constexpr int STEP_T = TILE_B / ROWB;            // tokens per step (8, 16 or 32)
  constexpr int NI = TILE_B / 1024;                // 1 KB direct loads per tile
  constexpr int RPI = 1024 / ROWB;                 // rows per direct load
  constexpr int NSTG = NW == 8 ? 2 : 4;            // ring stages per wave (same LDS either way)
  constexpr int MASK_OFF = 2 * TILE_B;             // stage: K, V, mask words
  constexpr int STAGE_B = 2 * TILE_B + 256;
  constexpr int OPS = 2 * NI + 1;                  // vector-memory operations per step
  constexpr int RING_B = NW * NSTG * STAGE_B;
  constexpr int RED_B = NW * R * (D + 2) * 4;
  static_assert(R <= kValuRows && R <= 64, "row capacity");
  static_assert(STEP_T <= 32 && 32 % STEP_T == 0, "a step's mask bits lie in one word");
  static_assert(RPI >= 2 && 32 % RPI == 0 && NI == 4, "staged-row permutation");
  using Shape = ValuShape<T, D, R>;
  static_assert(Shape::RING_B == RING_B && Shape::RED_B == RED_B, "shape constants agree");
  char* smem = lds;
  int32_t* tok_row = reinterpret_cast<int32_t*>(lds + Shape::TOK_OFF);

  const DevPlan& P = a.plan;
  const int g = bid % a.hkv;
  const int4 it0 = P.valu_items[2 * (bid / a.hkv)];
  const int4 it1 = P.valu_items[2 * (bid / a.hkv) + 1];
  const int32_t rb = it0.y, nr = it0.z, cs = it0.w;
  const int32_t len = it1.x, gofs = it1.y;
  const int W = P.mask_words;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tg = lane / LPT, li = lane % LPT;

  // queries of the rows (rows past nr repeat the last row; never stored)
  int32_t qrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) qrow[r] = P.slot_query[gofs + (rb + min(r, nr - 1)) / a.grp];
  // token rows as rows of this KV head (pool row * Hkv + g), permuted so a
  // lane's rows of one step are adjacent
  stage_token_rows<RPI, 64 * NW>(tok_row, P, a.block_table, cs, len, it1.w, a.hkv, g, [] {});
  // lane i loads the mask word of row i (rows past nr: the last row's)
  const int32_t mask_slot = gofs + (rb + min(lane, nr - 1)) / a.grp;
  const uint32_t* mask_src = P.slot_mask + static_cast<size_t>(mask_slot) * W;
  lds_barrier();

  char* ring = smem + w * NSTG * STAGE_B;
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  const int lrow = lane / CH, lch = lane % CH;     // this lane's row and 16-byte slot in each load
  // Row R of a tile stores chunk p ^ (R % RPI) in its slot p (R % RPI is the
  // loading lane's lrow for every load of the tile).
  const char* kbase = static_cast<const char*>(a.k) + (lch ^ lrow) * 16;
  const char* vbase = static_cast<const char*>(a.v) + (lch ^ lrow) * 16;
  const int nsteps = (len + STEP_T - 1) / STEP_T;
  const int my_steps = w < nsteps ? (nsteps - w + NW - 1) / NW : 0;

  // Loads of one step into one stage: NI K rows, NI V rows, the mask words.
  // Load n fetches rows n*RPI + lrow of the step (R = lrow + n*RPI, so
  // R % CH = lrow % CH for every n: one swizzle per lane); tokens past the
  // chunk end re-read its last token (finite values; masked).
  auto issue = [&](int i, int stage) {
    const int step = w + i * NW;
    const int base = step * STEP_T;
    const uint32_t sd = ring_lds + stage * STAGE_B;
    int32_t rows[NI];
    if (base + STEP_T <= len) {
      const int32_t* tr = tok_row + (base & ~31) + lrow * (32 / RPI) + (base & 31) / RPI;
      const int4 v4 = *reinterpret_cast<const int4*>(tr);
      rows[0] = v4.x; rows[1] = v4.y; rows[2] = v4.z; rows[3] = v4.w;
    } else {
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int t = min(base + n * RPI + lrow, len - 1);
        rows[n] = tok_row[(t & ~31) + (t % RPI) * (32 / RPI) + (t & 31) / RPI];
      }
    }
#pragma unroll
    for (int n = 0; n < NI; ++n)
      lds_dma16(kbase + static_cast<uint64_t>(static_cast<uint32_t>(rows[n])) * ROWB, sd + n * 1024);
#pragma unroll
    for (int n = 0; n < NI; ++n)
      lds_dma16(vbase + static_cast<uint64_t>(static_cast<uint32_t>(rows[n])) * ROWB, sd + TILE_B + n * 1024);
    lds_dma4(mask_src + (base >> 5), sd + MASK_OFF);
  };

  float m_run[R], m_true[R], l[R], o[R][EPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m_run[r] = kNegInf;
    m_true[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[r][e] = 0.f;
  }
  const float qscale = a.scale_log2;

  // The R Q rows go through the last ring stage (first refilled in step 0),
  // by direct-to-LDS loads like the KV rows, so no ordinary global load is
  // pending in the loop; then NSTG-1 steps are put in flight.
  constexpr int NQ = (R * ROWB + 1023) / 1024;     // Q loads of 1 KB
  static_assert(R * ROWB <= 2 * TILE_B, "Q rows fit in one stage");
  const uint32_t qstage = ring_lds + (NSTG - 1) * STAGE_B;
  if (my_steps > 0) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const int byte = n * 1024 + lane * 16;
      const int r = min(byte / ROWB, R - 1);       // lanes past R rows reload the last one
      const int row = rb + min(r, nr - 1);
      const int head = g * a.grp + row % a.grp;
      lds_dma16(static_cast<const char*>(a.q) + ((static_cast<int64_t>(qrow[r]) * a.hq + head) * D) * EB +
                    (byte % ROWB), qstage + n * 1024);
    }
  }
#pragma unroll
  for (int i = 0; i < NSTG - 1; ++i)
    if (i < my_steps) issue(i, i);
  constexpr int QW = LB / 4;   // 32-bit words of Q per lane and row
  uint32_t qv[R][QW];
  for (int i = 0; i < my_steps; ++i) {
    const int stage = i % NSTG;
    // this step's loads are done once at most the later issued steps remain
    const int later = min(NSTG - 2, my_steps - 1 - i);
    if (NSTG > 3 && later >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * OPS));
    else if (NSTG > 2 && later >= 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(OPS));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if (i == 0) {
      // Q rows (older than step 0's loads, so done too): bf16 stays packed
      // (scores by bf16 dot2, fp32 accumulate), fp32 as is
      const char* qs = ring + (NSTG - 1) * STAGE_B;
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(qs + r * ROWB + li * LB + j * 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) qv[r][4 * j + e] = raw[e];
        }
      }
      // the Q reads complete before this stage is refilled below
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    }
    // refill the stage read in step i-1 (its reads have all returned)
    if (i + NSTG - 1 < my_steps) issue(i + NSTG - 1, (i + NSTG - 1) % NSTG);
    const char* kb = ring + stage * STAGE_B;
    const int base = (w + i * NW) * STEP_T;
    const uint32_t* mw = reinterpret_cast<const uint32_t*>(kb + MASK_OFF);
    uint32_t mbits[R];
#pragma unroll
    for (int r = 0; r < R; ++r) mbits[r] = mw[r] >> (base & 31);
    // the step's K and V fragments for every pass, read before any is used
    constexpr int NPASS = STEP_T / TPW;
    u32x4 kfr[NPASS][NLD], vfr[NPASS][NLD];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int tr = ps * TPW + tg;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int sw = ((li * NLD + j) ^ (tr % RPI)) * 16;   // slot of chunk li * NLD + j
        kfr[ps][j] = *reinterpret_cast<const u32x4*>(kb + tr * ROWB + sw);
        vfr[ps][j] = *reinterpret_cast<const u32x4*>(kb + TILE_B + tr * ROWB + sw);
      }
    }
    if constexpr (EB == 2) {
      // bf16: the passes go in pairs, a lane's two tokens side by side.  V
      // element e of both sits in one dword (v_perm), the two probabilities
      // in one bf16x2, so each O accumulator (and l) takes one dot2 for two
      // tokens; P is rounded to bf16 as in the matrix-core path.
      static_assert(NPASS % 2 == 0, "passes come in pairs");
#pragma unroll
      for (int pp = 0; pp < NPASS; pp += 2) {
        const int tr0 = pp * TPW + tg, tr1 = tr0 + TPW;   // tokens within the step
        const bool valid0 = base + tr0 < len, valid1 = base + tr1 < len;
        uint32_t vp[EPL];
#pragma unroll
        for (int j = 0; j < NLD; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vp[j * 8 + 2 * i] = __builtin_amdgcn_perm(vfr[pp + 1][j][i], vfr[pp][j][i], 0x05040100u);
            vp[j * 8 + 2 * i + 1] = __builtin_amdgcn_perm(vfr[pp + 1][j][i], vfr[pp][j][i], 0x07060302u);
          }
        float z0[R], z1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int j = 0; j < NLD; ++j) {
            s0 = dot8_bf16(kfr[pp][j], qv[r] + 4 * j, s0);
            s1 = dot8_bf16(kfr[pp + 1][j], qv[r] + 4 * j, s1);
          }
          z0[r] = s0;
          z1[r] = s1;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          z0[r] = group_sum<LPT>(z0[r]) * qscale;
          z1[r] = group_sum<LPT>(z1[r]) * qscale;
        }
        bool raise[R];
        float zm[R];
        bool any_raise = false;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          z0[r] = valid0 && ((mbits[r] >> tr0) & 1u) ? z0[r] : kNegInf;
          z1[r] = valid1 && ((mbits[r] >> tr1) & 1u) ? z1[r] : kNegInf;
          zm[r] = fmaxf(z0[r], z1[r]);
          m_true[r] = fmaxf(m_true[r], zm[r]);
          raise[r] = zm[r] > m_run[r] + kRescaleSlack;
          any_raise |= raise[r];
        }
        if (__any(any_raise)) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float mn = raise[r] ? zm[r] : m_run[r];
            const float alpha = raise[r] ? fast_exp2(m_run[r] - mn) : 1.f;   // m = -inf gives 0
            m_run[r] = mn;
            l[r] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[r][e] *= alpha;
          }
        }
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        typedef float f32x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const bool none = m_run[r] == kNegInf;
          const float p0 = none ? 0.f : fast_exp2(z0[r] - m_run[r]);   // z = -inf gives 0
          const float p1 = none ? 0.f : fast_exp2(z1[r] - m_run[r]);
          const bf16x2_t pb = __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_t);
          l[r] = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l[r], false);
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            o[r][e] = __builtin_amdgcn_fdot2_f32_bf16(pb, __builtin_bit_cast(bf16x2_t, vp[e]), o[r][e], false);
        }
      }
    } else {
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
        const int tr = ps * TPW + tg;                 // token within the step
        const bool valid = base + tr < len;
        float vf[EPL];
#pragma unroll
        for (int j = 0; j < NLD; ++j) Elem<T>::unpack(vfr[ps][j], vf + j * (16 / EB));
        // All rows side by side (independent chains): scores, group sums,
        // mask, one branch for the rare rise of any running max, then the
        // probability and the O and l updates.
        float z[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float sc = 0.f;
#pragma unroll
          for (int e = 0; e < QW; ++e) sc = fmaf(__uint_as_float(qv[r][e]), __uint_as_float(kfr[ps][0][e]), sc);
          z[r] = sc;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) z[r] = group_sum<LPT>(z[r]) * qscale;
        bool raise[R];
        bool any_raise = false;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const bool vis = valid && ((mbits[r] >> tr) & 1u);
          z[r] = vis ? z[r] : kNegInf;
          m_true[r] = fmaxf(m_true[r], z[r]);
          // the running max rises only when a score exceeds it by the slack
          // (a running max of -inf is exceeded by any finite score)
          raise[r] = z[r] > m_run[r] + kRescaleSlack;
          any_raise |= raise[r];
        }
        if (__any(any_raise)) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float mn = raise[r] ? z[r] : m_run[r];
            const float alpha = raise[r] ? fast_exp2(m_run[r] - mn) : 1.f;   // m = -inf gives 0
            m_run[r] = mn;
            l[r] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[r][e] *= alpha;
          }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float p = m_run[r] == kNegInf ? 0.f : fast_exp2(z[r] - m_run[r]);   // z = -inf gives 0
          l[r] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
        }
      }
    }
  }

  // Merge the lane groups of this wave, then the waves (through LDS, over
  // the ring), at the true max.
  lds_barrier();
  float* red = reinterpret_cast<float*>(smem);   // [NW][R][D + 2]
#pragma unroll
  for (int r = 0; r < R; ++r) {
    auto add = [](float x, float y) { return x + y; };
    const float mx = cross_group_reduce<LPT>(m_true[r], [](float x, float y) { return fmaxf(x, y); });
    const float f = (m_run[r] == kNegInf) ? 0.f : fast_exp2(m_run[r] - mx);
    const float lsum = cross_group_reduce<LPT>(l[r] * f, add);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[r][e] = cross_group_reduce<LPT>(o[r][e] * f, add);
    if (tg == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[(w * R + r) * (D + 2) + li * EPL + e] = o[r][e];
      if (li == 0) {
        red[(w * R + r) * (D + 2) + D] = mx;
        red[(w * R + r) * (D + 2) + D + 1] = lsum;
      }
    }
  }
  lds_barrier();
  // two consecutive elements of one row per thread
  for (int idx = threadIdx.x; idx < nr * (D / 2); idx += blockDim.x) {
    const int r = idx / (D / 2), e = 2 * (idx % (D / 2));
    float mx = kNegInf;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) mx = fmaxf(mx, red[(ww * R + r) * (D + 2) + D]);
    float o0 = 0.f, o1 = 0.f, lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float* rw = red + (ww * R + r) * (D + 2);
      const float f = (rw[D] == kNegInf) ? 0.f : fast_exp2(rw[D] - mx);
      o0 = fmaf(f, rw[e], o0);
      o1 = fmaf(f, rw[e + 1], o1);
      lsum = fmaf(f, rw[D + 1], lsum);
    }
    const int row = rb + r;
    const int64_t sh = static_cast<int64_t>(gofs + row / a.grp) * a.hq + g * a.grp + row % a.grp;
    if (a.po_bf16) {
      const float inv = 1.f / lsum;
      st_u32<FUSED>(reinterpret_cast<uint16_t*>(a.po) + sh * D + e, pack_bf16x2(o0 * inv, o1 * inv));
    } else {
      st_u32x2<FUSED>(a.po + sh * D + e, __float_as_uint(o0), __float_as_uint(o1));
    }
    if (e == 0) {
      st_f32<FUSED>(a.pm + sh, mx == kNegInf ? kNegInf : mx * kLn2);
      st_f32<FUSED>(a.pl + sh, lsum);
    }
  }
  if constexpr (FUSED) {
    fused_publish<kValuRows>(P, a.hq, a.grp, rb, nr, gofs, g);
  }
}

// ---------------------------------------------------------------------------
// MFMA partial kernel (bf16).  Work-group = 8 waves (two per SIMD) on one
// (chunk, KV head, block of up to 64 rows).  Wave w owns row half h = w & 1
// (rows 32h .. 32h+31, two 16-row tiles) and token split sp = w >> 1: it takes
// the chunk's 32-token steps sp, sp+4, ...  The two waves of a split share a
// two-stage LDS ring; per step one of them loads the K rows and the 64 rows'
// mask words, the other the V rows, by direct-to-LDS loads (no VGPRs), one
// step ahead; the two rendezvous through LDS flags once per step (no
// work-group barrier inside the loop).  Per step and wave:
//   S^T = K Q^T   16x16x32 MFMA, A = K rows (LDS), B = Q^T (registers), for
//                 2 token tiles x 2 row tiles;
//   mask, online softmax on the S^T fragments in registers;
//   O^T += V^T P^T  A = V^T from LDS transpose reads of the token-major V
//                 rows, B = P^T taken straight from the S^T fragments; the
//                 row sums l by the same product with a tile of ones as A.
// K tile rows are permuted so every lane ends up holding 8 consecutive tokens
// of one row, which is the B-operand layout of the PV product.  Rows in LDS
// are stored with their 16-byte chunks XOR-swizzled by the row index.  The
// four token splits of each row half are merged through LDS at the end.
// Wide items (NSPLIT = 2) cover 128 rows instead: four 32-row groups per
// split (gr = w % 4, sp = w / 4) share each split's ring and its loads (a
// quarter each), rendezvous through four flags, and split 1's results are
// merged into split 0's registers at the end.
// ---------------------------------------------------------------------------
// Swizzle of the 16-byte chunks of a KV or Q row in LDS: slot p of LDS row R
// holds chunk p ^ kv_swz<CH>(R) (CH chunks per row).  For 256-byte rows the
// key is built from bits 0-1 and 3-4 of R, with bit 2 flipping its top bit:
// the 16 lanes that share a K fragment read (rows 8a + b + 4c, a, b = 0..3,
// c fixed) then hit 16 distinct slots, so the ds_read_b128 runs without bank
// conflicts (measured on gfx950: 198 B/clk per CU against 117 for R % 16),
// while the V transpose reads keep their rate.  For 128-byte rows, R % 8.
// The key has a period of kSwzRows<CH> rows.
template <int CH>
__device__ constexpr int kv_swz(int R) {
  if constexpr (CH == 16) return ((R & 3) | (((R >> 3) & 3) << 2)) ^ (((R >> 2) & 1) << 3);
  else return R % CH;
}
template <int CH>
constexpr int kSwzRows = CH == 16 ? 32 : CH;

template <int D, int NSPLIT>
struct MfmaShape {
  static constexpr int NGRP = 8 / NSPLIT;        // waves sharing a split's ring
  static constexpr int ROWS = 32 * NGRP;         // rows of a work item
  static constexpr int ROWB = D * 2;
  static constexpr int TILE_B = 32 * ROWB;
  static constexpr int STAGE_B = 2 * TILE_B + 4 * ROWS;   // K, V, a mask word per row
  static constexpr int RING_B = NSPLIT * 2 * STAGE_B;
  // LDS carve-out: rings (and the epilogue's reduction), the Q rows (in
  // stage 1 of split 0 with four splits, a region of their own with two),
  // staged token rows, split statistics, group flags, fused-merge lists
  static constexpr int QOFF = NSPLIT == 4 ? STAGE_B : RING_B;
  static constexpr int TOK_OFF = NSPLIT == 4 ? RING_B : RING_B + ROWS * ROWB;
  static constexpr int STATS_OFF = TOK_OFF + 4 * kMaxChunkTokens;
  static constexpr int FLAGS_OFF = STATS_OFF + 8 * 32 * 3 * 4;
  static constexpr int LDS_B = FLAGS_OFF + 4 * 8;
  static_assert(FLAGS_OFF % 16 == 0, "a split's flags are read as one 16-byte word");
};

template <int D, bool FUSED, int NSPLIT>
__device__ __forceinline__ void mfma_body(const PartialArgs& a, char* lds, int bid, int item_base) {
  constexpr int NWAVE = 8;
  constexpr int NGRP = NWAVE / NSPLIT;  // waves per split, one per 32-row group
  constexpr int NRT = 2;                // row tiles per wave
  constexpr int WROWS = NRT * 16;       // rows per wave
  constexpr int ROWS = NGRP * WROWS;    // rows of the work item
  constexpr int KS = D / 32;            // k-steps of S = K Q^T
  constexpr int DT = D / 16;            // d-tiles of O^T
  constexpr int CH = D / 8;             // 16-byte chunks per token row
  constexpr int ROWB = D * 2;           // bytes per token row
  constexpr int TILE_B = 32 * ROWB;     // K (or V) bytes of one 32-token step
  constexpr int NI = TILE_B / 1024;     // 1 KB direct loads per tile
  constexpr int RPI = 64 / CH;          // token rows per direct load
  constexpr int STAGE_B = 2 * TILE_B + 4 * ROWS;   // K, V, a mask word per row
  constexpr int RING_B = NSPLIT * 2 * STAGE_B;
  constexpr int RED_W = DT * NRT * 64 * 16;   // one wave's O^T fragments (epilogue)
  // A step's loads are shared by the NGRP waves of a split: NL direct loads
  // each (the K tile's, then the V tile's, in order), and the mask words of
  // 64 rows for each of the first ROWS / 64 waves.
  constexpr int NL = 2 * NI / NGRP;
  static_assert(NI == 8 || NI == 4, "token rows per lane come in groups of 4 or 8");
  static_assert(NSPLIT == 4 || NSPLIT == 2, "64-row items in four splits, 128-row items in two");
  static_assert(NL >= 2 && (NL == NI || 2 * NL == NI), "whole halves of a tile per wave");
  using Shape = MfmaShape<D, NSPLIT>;
  static_assert(Shape::RING_B == RING_B && Shape::STAGE_B == STAGE_B && Shape::ROWS == ROWS, "shape constants agree");
  static_assert(NSPLIT == 2 || 2 * RED_W <= 2 * STAGE_B, "a split's two waves reduce through their own ring");
  static_assert(NSPLIT == 4 || (2 * RED_W <= ROWS * ROWB && 2 * RED_W <= 2 * STAGE_B),
                "split 1's waves publish through the Q region and their own ring");
  char* smem = lds;
  int32_t* tok_row = reinterpret_cast<int32_t*>(lds + Shape::TOK_OFF);
  float (*stats)[WROWS][3] = reinterpret_cast<float (*)[WROWS][3]>(lds + Shape::STATS_OFF);
  int32_t (*grp_ready)[NGRP] = reinterpret_cast<int32_t (*)[NGRP]>(lds + Shape::FLAGS_OFF);

  const DevPlan& P = a.plan;
  const int g = bid % a.hkv;
  const int item = item_base + bid / a.hkv;
  const int4 it0 = P.mfma_items[2 * item];
  const int4 it1 = P.mfma_items[2 * item + 1];
  const int32_t rb = it0.y, nr = it0.z, cs = it0.w;
  const int32_t len = it1.x, gofs = it1.y;
  const bool full = it1.z != 0;
  const int W = P.mask_words;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gr = w % NGRP, sp = w / NGRP;   // row group (rows 32 gr ..) and token split
  const int kvsel = gr * NL / NI;           // this wave loads K (0) or V (1) rows
  const int n0 = gr * NL % NI;              // its first load of that tile
  const bool loads_mask = gr < ROWS / 64;
  const int lr = lane & 15, lj = lane >> 4;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* vp = static_cast<const uint16_t*>(a.v);

  // The block's Q rows (ROWS * 2D bytes) are copied once into LDS: into
  // stage 1 of split 0's ring with four splits (first refilled in the loop,
  // after every wave has read its fragments), into a region of their own with
  // two.  Copy n (1 KB, NQW per wave) holds rows RPQ*n
  // .. RPQ*n + RPQ-1; its lane i takes 16-byte chunk (i % CH) ^ kv_swz(R) of
  // row R = RPQ*n + i / CH, so the fragment reads below avoid bank
  // conflicts.  The rows' queries are looked up alongside the flat-to-logical
  // lookups of the staging, the copies are issued alongside its block-table
  // lookups.  Rows past nr copy a valid row; they are masked later.
  constexpr int RPQ = 1024 / ROWB;
  constexpr int NQW = ROWS * ROWB / 1024 / NWAVE;
  static_assert(NSPLIT == 2 || ROWS * ROWB <= STAGE_B, "the block's Q rows fit in one ring stage");
  static_assert(NQW >= 1 && NQW * NWAVE * 1024 == ROWS * ROWB, "whole 1 KB Q copies per wave");
  const uint32_t q_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem + Shape::QOFF));
  int32_t qsq[NQW];
#pragma unroll
  for (int j = 0; j < NQW; ++j) {
    const int R = RPQ * (NQW * w + j) + lane / CH;
    qsq[j] = P.slot_query[gofs + (rb + min(R, nr - 1)) / a.grp];
  }
  // token rows are stored as rows of this KV head: pool row * Hkv + g
  stage_token_rows<RPI, 512>(tok_row, P, a.block_table, cs, len, it1.w, a.hkv, g, [&] {
#pragma unroll
    for (int j = 0; j < NQW; ++j) {
      const int R = RPQ * (NQW * w + j) + lane / CH;
      const int row = rb + min(R, nr - 1);
      const int head = g * a.grp + row % a.grp;
      const int c = (lane % CH) ^ kv_swz<CH>(R);
      lds_dma16(qp + (static_cast<int64_t>(qsq[j]) * a.hq + head) * D + c * 8, q_lds + (NQW * w + j) * 1024);
    }
  });
  // Row of the mask word this lane loads (lane i <-> row 64 gr + i of the
  // block, for the waves that load mask words).
  const int mrow = 64 * (loads_mask ? gr : 0) + lane;
  const int32_t mask_slot = gofs + (rb + (mrow < nr ? mrow : 0)) / a.grp;
  if (threadIdx.x < NSPLIT * NGRP) grp_ready[threadIdx.x / NGRP][threadIdx.x % NGRP] = -1;
  lds_barrier();   // the staged token rows are visible (the Q copies may still be in flight)

  char* ring = smem + sp * 2 * STAGE_B;
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  const int lrow = lane / CH;            // row of each direct load this lane fetches
  const int lch = lane % CH;             // its 16-byte LDS slot in that row

  // This wave's share of a step's loads: loads n0 .. n0 + NL - 1 of the K
  // (kvsel = 0) or V tile, and mask words.  Load n fetches rows n*RPI + lrow;
  // lane (lrow, lch) fetches chunk lch ^ kv_swz(R) of row R, so LDS slot p of
  // row R holds chunk p ^ kv_swz(R).  Each lane keeps one base pointer per
  // load of its share (the swizzle of its row in that load), so a load
  // address is one shift-add of the staged head row.
  // Tokens past the chunk end re-read its last token (finite values; masked).
  static_assert(NI * RPI == 32 && 32 % kSwzRows<CH> == 0, "the swizzle repeats within a 32-token step");
  const char* lbase[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j)
    lbase[j] = reinterpret_cast<const char*>(kvsel ? vp : kp) + (lch ^ kv_swz<CH>((n0 + j) * RPI + lrow)) * 16;
  auto load_ptrs = [&](int step, const char** ptr) {
    // (the staged rows run to a multiple of 512 tokens, entries past the
    // chunk end holding its last token, so a partial last step needs no
    // special case)
    int32_t rows[NL];
    const int32_t* tr = tok_row + step * 32 + lrow * NI + n0;   // the permuted layout
    if constexpr (NL >= 4) {
#pragma unroll
      for (int j = 0; j < NL; j += 4) {
        const int4 v4 = *reinterpret_cast<const int4*>(tr + j);
        rows[j] = v4.x; rows[j + 1] = v4.y; rows[j + 2] = v4.z; rows[j + 3] = v4.w;
      }
    } else {
      const int2 v2 = *reinterpret_cast<const int2*>(tr);
      rows[0] = v2.x; rows[1] = v2.y;
    }
#pragma unroll
    for (int j = 0; j < NL; ++j)
      ptr[j] = lbase[j] + (static_cast<uint64_t>(static_cast<uint32_t>(rows[j])) * ROWB);
  };
  const uint32_t* mask_src = P.slot_mask + static_cast<size_t>(mask_slot) * W;

  f32x4 o[DT][NRT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Per row tile: the running max m_run (raw score units) with its exp2
  // offset mc = m_run * scale * log2(e) and rescale threshold thr, both
  // updated only when m_run rises; the lane's true max; and the row sum of
  // P, accumulated by the matrix core against a tile of ones (every element
  // of lacc[rt] holds the sum of the lane's row).
  const float cl2 = a.scale_log2;
  float m_run[NRT], m_true[NRT], mc[NRT], thr[NRT];
  f32x4 lacc[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m_run[rt] = kNegInf;
    m_true[rt] = kNegInf;
    mc[rt] = 0.f;
    thr[rt] = kNegInf;
    lacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int nsteps = (len + 31) / 32;
  const int iters = (nsteps + NSPLIT - 1) / NSPLIT;   // the same for every wave
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;

  // LDS byte offsets (from the block's LDS base: stage 0 of this split's
  // ring; stage 1 adds STAGE_B as an immediate) of this lane's operand
  // fragments: K fragment n = (ks, tt) for S, and the two halves of V^T
  // d-tile dt for PV.
  const int rk0 = 8 * (lr >> 2) + (lr & 3);   // K rows of this lane, per token tile
  int koff[2 * KS], voff[DT][2];
#pragma unroll
  for (int n = 0; n < 2 * KS; ++n) {
    const int ks = n >> 1, R = rk0 + 4 * (n & 1);
    koff[n] = sp * 2 * STAGE_B + R * ROWB + (((ks * 4 + lj) ^ kv_swz<CH>(R)) * 16);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int R = 8 * lj + 4 * hh + (lr >> 2);
      voff[dt][hh] = sp * 2 * STAGE_B + TILE_B + R * ROWB + (((2 * dt + ((lr & 3) >> 1)) ^ kv_swz<CH>(R)) * 16) +
                     8 * (lr & 1);
    }

  // The split's first step goes out before waiting for the Q copies; then
  // each wave waits for its own Q copies only (they are older than the step's
  // loads) and a barrier makes all of them visible.
  if (sp < nsteps) {
    const char* ptr[NL];
    load_ptrs(sp, ptr);
#pragma unroll
    for (int j = 0; j < NL; ++j) lds_dma16(ptr[j], ring_lds + kvsel * TILE_B + (n0 + j) * 1024);
    if (loads_mask) {
      lds_dma4(mask_src + sp, ring_lds + 2 * TILE_B + gr * 256);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL + 1));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL));
    }
  } else {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
  lds_barrier();
  // Q^T fragments (B operand of S^T = K Q^T) of this wave's 32 rows: lane
  // (lr, lj) takes d = 32 ks + 8 lj .. +7 of row R = 32gr + 16rt + lr, i.e.
  // chunk 4 ks + lj, stored in slot (4 ks + lj) ^ kv_swz(R).  Every wave reads
  // them before any wave refills stage 1 of split 0 (the barrier below; this
  // step's loads above go to stage 0).
  bf16x8 qf[NRT][KS];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int R = WROWS * gr + rt * 16 + lr;
      qf[rt][ks] = *reinterpret_cast<const bf16x8*>(smem + Shape::QOFF + R * ROWB + (((4 * ks + lj) ^ kv_swz<CH>(R)) * 16));
    }
  lds_barrier();

  // One step on ring stage STG (a compile-time constant, so every LDS address
  // is a per-lane base plus an immediate offset).
  // A operand of the row-sum product: 16 rows of ones.
  const bf16x8 ones8 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f),
                        static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f),
                        static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  auto step_body = [&](auto stg, int i) {
    constexpr int STG = decltype(stg)::value;
    const int step = sp + i * NSPLIT;
    // This wave's loads for `step` are done.  Only the waves of a split
    // share a ring, so they synchronise with each other instead of the whole
    // work-group: each publishes "my share of iteration i is in LDS and I
    // have finished iteration i-1", then waits for the others to say the
    // same, after which the other stage can be refilled with step i+1.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    group_sync<NGRP>(grp_ready[sp], gr, i, lane, a.spin_limit, P.status);
    if (step >= nsteps) return;
    const bool next = step + NSPLIT < nsteps;
    const int base = step * 32;
    const char* kb = ring + STG * STAGE_B;
    const uint32_t* mb = reinterpret_cast<const uint32_t*>(kb + 2 * TILE_B);
    const uint32_t nd = ring_lds + (STG ^ 1) * STAGE_B + kvsel * TILE_B;   // this wave's tile in the other stage
    // The step runs row tile by row tile so that each tile's softmax
    // arithmetic is issued between the MFMAs of the next product (S of tile
    // 1, then PV of tile 0) and executes while the matrix unit works:
    //   S(0) | softmax(0) max  | S(1) + softmax(0) exp | softmax(1) max |
    //   PV(0) + softmax(1) exp | PV(1)
    // Waves keep a raised issue priority for the whole step.  The K
    // fragment reads go out first, then the next step's loads (their
    // address arithmetic runs while the fragments arrive; the MFMA runs
    // stay free of branches, so the arithmetic can be interleaved with them).
    bf16x8 kfr[2 * KS];
#pragma unroll
    for (int n = 0; n < 2 * KS; ++n) kfr[n] = *reinterpret_cast<const bf16x8*>(smem + STG * STAGE_B + koff[n]);
    if (next) {
      const char* ptr[NL];
      load_ptrs(step + NSPLIT, ptr);
#pragma unroll
      for (int j = 0; j < NL; ++j) lds_dma16(ptr[j], nd + (n0 + j) * 1024);
      if (loads_mask) lds_dma4(mask_src + step + NSPLIT, ring_lds + (STG ^ 1) * STAGE_B + 2 * TILE_B + gr * 256);
    }
    __builtin_amdgcn_s_setprio(1);
    // S^T = K Q^T for row tile rt: sacc[tt][rt] over the 4 k-steps; n = (ks, tt).
    f32x4 sacc[2][NRT];
    auto s_tile = [&](auto rtc) {
      constexpr int rt = decltype(rtc)::value;
#pragma unroll
      for (int n = 0; n < 2 * KS; ++n) {
        sacc[n & 1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            kfr[n], qf[rt][n >> 1], n < 2 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[n & 1][rt], 0, 0, 0);
      }
    };
    s_tile(std::integral_constant<int, 0>{});

    // V^T fragments for the PV product, read now so their LDS latency is
    // hidden.  They come from transpose reads of the token-major rows:
    // within each 16-lane group, ds_read_b64_tr_b16 hands lane i element
    // (i % 4) of the 8 bytes that lane 4k + i/4 addresses, as its k-th
    // element.  Lane (lr, lj) addresses row 8lj + 4h' + lr/4 at d
    // 16dt + 4(lr % 4), so it receives V[8lj + 4h' + k][16dt + lr], k = 0..3.
    bf16x8 vfr[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x2 half[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        half[hh] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                       (lds_s16x4_t)(smem + STG * STAGE_B + voff[dt][hh])));
      vfr[dt] = __builtin_bit_cast(bf16x8, u32x4{half[0][0], half[0][1], half[1][0], half[1][1]});
    }

    // Mask and online softmax.  Lane holds tokens base + 8*lj + e of row
    // 32h + rt*16 + lr; scores stay in raw units, exp2 folds in scale*log2(e).
    // The running max m_run of a row (shared by its 4 lanes) only rises when
    // some lane sees a score above m_run + slack; only then are the 4 lanes
    // reduced.  The true max is tracked per lane and reduced at the end.  l
    // sums the probabilities as rounded to bf16 for the PV product.
    bf16x8 pb[NRT];
    float z[NRT][8];
    const int valid_e = len - base - 8 * lj;   // tokens of this lane's 8 that exist
    const bool all_visible = full && valid_e >= 8;
    auto soft_max = [&](auto rtc) {       // mask, maxima, lazy rescale
      constexpr int rt = decltype(rtc)::value;
      const int rl = WROWS * gr + rt * 16 + lr;   // row within the block
      const bool row_ok = rl < nr;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[rt][e] = e < 4 ? sacc[0][rt][e] : sacc[1][rt][e - 4];
      if (!all_visible) {
        const uint32_t bits = row_ok ? (mb[rl] >> (8 * lj)) & 0xffu : 0u;
        // a step of a partly masked chunk whose tokens every row of the tile
        // sees (the prefix part of a chunk that also holds tree tokens) needs
        // no selects
        if (!__all(bits == 0xffu && valid_e >= 8)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) z[rt][e] = (((bits >> e) & 1u) && e < valid_e) ? z[rt][e] : kNegInf;
        }
      } else if (!row_ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) z[rt][e] = kNegInf;
      }
      float mx = z[rt][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[rt][e]);
      m_true[rt] = fmaxf(m_true[rt], mx);
      // (a running max of -inf is exceeded by any finite score)
      const bool high = mx > thr[rt];
      if (__any(high)) {
        const float rmx = rowmax4(mx);
        const bool raise = rmx > thr[rt];
        const float mn = raise ? rmx : m_run[rt];
        const float alpha = raise ? fast_exp2((m_run[rt] - mn) * cl2) : 1.f;
        m_run[rt] = mn;
        mc[rt] = mn == kNegInf ? 0.f : mn * cl2;
        thr[rt] = mn + kRescaleSlack / cl2;
        lacc[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
      }
    };
    auto soft_exp = [&](auto rtc) {       // probabilities, bf16 P
      constexpr int rt = decltype(rtc)::value;
      // (a row with nothing visible yet has mc = 0 and z all -inf)
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(z[rt][e], cl2, -mc[rt]));   // z = -inf gives 0
      pb[rt] = __builtin_convertvector(p, bf16x8);
    };
    // O^T += V^T P^T for row tile rt, and l += 1 P^T (the sums of the
    // probabilities as rounded to bf16 for the product).
    auto pv_tile = [&](auto rtc) {
      constexpr int rt = decltype(rtc)::value;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr[dt], pb[rt], o[dt][rt], 0, 0, 0);
      }
      lacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pb[rt], lacc[rt], 0, 0, 0);
    };
    // one MFMA, then up to three VALU instructions, for each MFMA of the run
    auto interleave = [] {
#pragma unroll
      for (int k = 0; k < DT; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
    };
    static_assert(NRT == 2 && 2 * KS == DT, "the schedule is written for two row tiles");
    soft_max(std::integral_constant<int, 0>{});
    s_tile(std::integral_constant<int, 1>{});
    soft_exp(std::integral_constant<int, 0>{});
    interleave();
    // keep tile 0's probabilities here (the compiler would otherwise sink
    // them past tile 1's branches, next to their use)
    asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pb[0])));
    soft_max(std::integral_constant<int, 1>{});
    pv_tile(std::integral_constant<int, 0>{});
    soft_exp(std::integral_constant<int, 1>{});
    interleave();
    pv_tile(std::integral_constant<int, 1>{});
    __builtin_amdgcn_s_setprio(0);
  };
  for (int i = 0; i < iters; i += 2) {
    step_body(std::integral_constant<int, 0>{}, i);
    if (i + 1 < iters) step_body(std::integral_constant<int, 1>{}, i + 1);
  }

  // Combine the four token splits of each row half.  Each wave publishes its
  // rows' (running max, true max, l) and its unscaled O^T fragments as f32x4
  // at red[dt][rt][lane] in its half of its own split's ring, as soon as its
  // partner is done with that ring too, so waves that finish early write
  // while others still compute.  After one barrier every thread takes DT/2
  // d-tiles of one row: M = the splits' largest true max, weights
  // f_q = exp2(m_run_q - M), l = sum f_q l_q, O = sum f_q O_q.
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float ls = lacc[rt][0];
    const float mt = rowmax4(m_true[rt]);
    if (lj == 0) {
      stats[w][rt * 16 + lr][0] = m_run[rt];
      stats[w][rt * 16 + lr][1] = mt;
      stats[w][rt * 16 + lr][2] = ls;
    }
  }
  if constexpr (NSPLIT == 4) {
    group_sync<NGRP>(grp_ready[sp], gr, iters, lane, a.spin_limit, P.status);   // the split is past its last step
    {
      f32x4* mine = reinterpret_cast<f32x4*>(smem + sp * 2 * STAGE_B + gr * RED_W);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) mine[(dt * NRT + rt) * 64 + lane] = o[dt][rt];
    }
    lds_barrier();
    {
      static_assert(NGRP == 2 && 2 * NRT * 64 * 2 == 512, "thread -> (d half, row half, row tile, lane)");
      const int ln = threadIdx.x & 63, rt = (threadIdx.x >> 6) % NRT;
      const int hh = (threadIdx.x >> 6) / NRT % 2, dq = threadIdx.x >> 8;
      const int rw = rt * 16 + (ln & 15), r = WROWS * hh + rw;
      float mx = kNegInf;
#pragma unroll
      for (int q = 0; q < NSPLIT; ++q) mx = fmaxf(mx, stats[2 * q + hh][rw][1]);
      float f[NSPLIT], ls = 0.f;
#pragma unroll
      for (int q = 0; q < NSPLIT; ++q) {
        const float mr = stats[2 * q + hh][rw][0];
        f[q] = (mr == kNegInf) ? 0.f : fast_exp2((mr - mx) * cl2);
        ls += f[q] * stats[2 * q + hh][rw][2];
      }
      if (r < nr) {
        const int row = rb + r;
        const int64_t sh = static_cast<int64_t>(gofs + row / a.grp) * a.hq + g * a.grp + row % a.grp;
        if (ln < 16 && dq == 0) {
          st_f32<FUSED>(a.pm + sh, mx == kNegInf ? kNegInf : mx * cl2 * kLn2);
          st_f32<FUSED>(a.pl + sh, ls);
        }
        const float inv = 1.f / ls;
#pragma unroll
        for (int k = 0; k < DT / 2; ++k) {
          const int dt = dq * (DT / 2) + k;
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < NSPLIT; ++q)
            acc += f[q] * reinterpret_cast<const f32x4*>(smem + q * 2 * STAGE_B + hh * RED_W)[(dt * NRT + rt) * 64 + ln];
          const int64_t at = sh * D + dt * 16 + (ln >> 4) * 4;
          if (a.po_bf16) {
            const uint32_t lo = pack_bf16x2(acc[0] * inv, acc[1] * inv);
            const uint32_t hi = pack_bf16x2(acc[2] * inv, acc[3] * inv);
            st_u32x2<FUSED>(reinterpret_cast<uint16_t*>(a.po) + at, lo, hi);
          } else {
            st_f32x4<FUSED>(a.po + at, acc);
          }
        }
      }
    }
  } else {
    // Two splits: split 1's waves publish their O^T fragments once their
    // split is past its last step, row groups 0 and 1 in the Q region (free
    // since the prologue), 2 and 3 in their own ring; after one barrier each
    // split-0 wave merges its partner's rows (same row group) into its own
    // registers and writes them.
    auto red_of = [&](int grp) {
      return reinterpret_cast<f32x4*>(smem + (grp < 2 ? Shape::QOFF + grp * RED_W : 2 * STAGE_B + (grp - 2) * RED_W));
    };
    if (sp == 1) {
      group_sync<NGRP>(grp_ready[1], gr, iters, lane, a.spin_limit, P.status);
      f32x4* mine = red_of(gr);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) mine[(dt * NRT + rt) * 64 + lane] = o[dt][rt];
    }
    lds_barrier();
    if (sp == 0) {
      const int pw = NGRP + gr;   // the split-1 wave of this row group
      const f32x4* theirs = red_of(gr);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int rw = rt * 16 + lr, r = WROWS * gr + rw;
        const float m1 = stats[pw][rw][0];
        const float mx = fmaxf(stats[w][rw][1], stats[pw][rw][1]);
        const float f0 = m_run[rt] == kNegInf ? 0.f : fast_exp2((m_run[rt] - mx) * cl2);
        const float f1 = m1 == kNegInf ? 0.f : fast_exp2((m1 - mx) * cl2);
        const float ls = f0 * stats[w][rw][2] + f1 * stats[pw][rw][2];
        if (r < nr) {
          const int row = rb + r;
          const int64_t sh = static_cast<int64_t>(gofs + row / a.grp) * a.hq + g * a.grp + row % a.grp;
          if (lj == 0) {
            st_f32<FUSED>(a.pm + sh, mx == kNegInf ? kNegInf : mx * cl2 * kLn2);
            st_f32<FUSED>(a.pl + sh, ls);
          }
          const float inv = 1.f / ls;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const f32x4 acc = f0 * o[dt][rt] + f1 * theirs[(dt * NRT + rt) * 64 + lane];
            const int64_t at = sh * D + dt * 16 + lj * 4;
            if (a.po_bf16) {
              const uint32_t lo = pack_bf16x2(acc[0] * inv, acc[1] * inv);
              const uint32_t hi = pack_bf16x2(acc[2] * inv, acc[3] * inv);
              st_u32x2<FUSED>(reinterpret_cast<uint16_t*>(a.po) + at, lo, hi);
            } else {
              st_f32x4<FUSED>(a.po + at, acc);
            }
          }
        }
      }
    }
  }
  if constexpr (FUSED) {
    fused_publish<ROWS>(P, a.hq, a.grp, rb, nr, gofs, g);
  }
}

// ---------------------------------------------------------------------------
// MFMA partial kernel for whole groups (bf16): one work-group takes every
// row of a chunk's group for one KV head, up to 256 rows (8 waves of 32 rows,
// two 16-row tiles each), and streams the chunk's KV into LDS once for all of
// them ("1. KV-Guided Grouping": the group's KV is loaded on chip once and
// every grouped query scores against it).  There is no token split: every
// wave runs every 32-token step of the chunk on its own rows, so a wave's
// (O, m, l) is final after the loop and is written straight from registers
// (no merge through LDS, no wait for a slower split).  The 8 waves share one
// NSTG-stage LDS ring filled NSTG-1 steps ahead by direct-to-LDS loads, each
// wave loading 1/8 of a step's K and V rows (and, for waves 0-3, the mask
// words of 64 rows); one work-group barrier per step both publishes step i's
// loads and frees the stage read in step i-1.  The arithmetic of a step
// (S^T = K Q^T, mask, online softmax with the lazily raised running max, O^T
// += V^T P^T, row sums on the matrix core) is that of mfma_body.
// ---------------------------------------------------------------------------
template <int D>
struct MfmaGroupShape {
  static constexpr int NWAVE = 8;
  static constexpr int ROWS = 32 * NWAVE;        // rows of a work item
  static constexpr int NSTG = 4;                 // ring stages (NSTG - 1 steps ahead)
  static constexpr int ROWB = D * 2;
  static constexpr int TILE_B = 32 * ROWB;
  static constexpr int STAGE_B = 2 * TILE_B + 4 * ROWS;   // K, V, a mask word per row
  static constexpr int RING_B = NSTG * STAGE_B;
  // LDS carve-out: ring, the block's Q rows, staged token rows, fused-merge lists
  static constexpr int QOFF = RING_B;
  static constexpr int TOK_OFF = QOFF + ROWS * ROWB;
  static constexpr int LDS_B = TOK_OFF + 4 * kMaxChunkTokens;
};

template <int D, bool FUSED>
__device__ __forceinline__ void mfma_group_body(const PartialArgs& a, char* lds, int bid, int item_base) {
  using Shape = MfmaGroupShape<D>;
  constexpr int NWAVE = Shape::NWAVE;
  constexpr int NSTG = Shape::NSTG;
  constexpr int NRT = 2;                // row tiles per wave
  constexpr int WROWS = NRT * 16;       // rows per wave
  constexpr int ROWS = Shape::ROWS;
  constexpr int KS = D / 32;            // k-steps of S = K Q^T
  constexpr int DT = D / 16;            // d-tiles of O^T
  constexpr int CH = D / 8;             // 16-byte chunks per token row
  constexpr int ROWB = Shape::ROWB;
  constexpr int TILE_B = Shape::TILE_B;
  constexpr int STAGE_B = Shape::STAGE_B;
  constexpr int NI = TILE_B / 1024;     // 1 KB direct loads per tile
  constexpr int RPI = 64 / CH;          // token rows per direct load
  constexpr int NL = 2 * NI / NWAVE;    // direct loads per wave and step
  constexpr int MASK_WAVES = ROWS / 64; // waves that also load 64 rows' mask words
  static_assert(NL >= 1 && NL * NWAVE == 2 * NI, "a step's K and V loads split evenly over the waves");
  static_assert(NI % NL == 0, "a wave's loads lie in one tile");
  static_assert(Shape::LDS_B <= 160 * 1024, "LDS carve-out");
  char* smem = lds;
  int32_t* tok_row = reinterpret_cast<int32_t*>(lds + Shape::TOK_OFF);

  const DevPlan& P = a.plan;
  const int g = bid % a.hkv;
  const int item = item_base + bid / a.hkv;
  const int4 it0 = P.mfma_items[2 * item];
  const int4 it1 = P.mfma_items[2 * item + 1];
  const int32_t rb = it0.y, nr = it0.z, cs = it0.w;
  const int32_t len = it1.x, gofs = it1.y;
  const bool full = it1.z != 0;
  const int W = P.mask_words;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kvsel = w * NL / NI;        // this wave loads K (0) or V (1) rows
  const int n0 = w * NL % NI;           // its first load of that tile
  const bool loads_mask = w < MASK_WAVES;
  const bool active = WROWS * w < nr;   // the wave has rows to compute
  const int lr = lane & 15, lj = lane >> 4;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* vp = static_cast<const uint16_t*>(a.v);

  // The block's Q rows (ROWS * 2D bytes) are copied once into their own LDS
  // region, 1 KB per copy (NQW per wave): copy n holds rows RPQ*n ..
  // RPQ*n + RPQ-1, its lane i taking 16-byte chunk (i % CH) ^ kv_swz(R) of row
  // R = RPQ*n + i / CH.  The rows' queries are looked up alongside the
  // staging's flat-to-logical lookups and the copies issued alongside its
  // block-table lookups.  Rows past nr copy a valid row (masked later).
  constexpr int RPQ = 1024 / ROWB;
  constexpr int NQW = ROWS * ROWB / 1024 / NWAVE;
  static_assert(NQW >= 1 && NQW * NWAVE * 1024 == ROWS * ROWB, "whole 1 KB Q copies per wave");
  const uint32_t q_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem + Shape::QOFF));
  int32_t qsq[NQW];
#pragma unroll
  for (int j = 0; j < NQW; ++j) {
    const int R = RPQ * (NQW * w + j) + lane / CH;
    qsq[j] = P.slot_query[gofs + (rb + min(R, nr - 1)) / a.grp];
  }
  // token rows are stored as rows of this KV head: pool row * Hkv + g
  stage_token_rows<RPI, 512>(tok_row, P, a.block_table, cs, len, it1.w, a.hkv, g, [&] {
#pragma unroll
    for (int j = 0; j < NQW; ++j) {
      const int R = RPQ * (NQW * w + j) + lane / CH;
      const int row = rb + min(R, nr - 1);
      const int head = g * a.grp + row % a.grp;
      const int c = (lane % CH) ^ kv_swz<CH>(R);
      lds_dma16(qp + (static_cast<int64_t>(qsq[j]) * a.hq + head) * D + c * 8, q_lds + (NQW * w + j) * 1024);
    }
  });
  // Row of the mask word this lane loads (lane i <-> row 64 w + i).
  const int mrow = 64 * (loads_mask ? w : 0) + lane;
  const int32_t mask_slot = gofs + (rb + (mrow < nr ? mrow : 0)) / a.grp;
  const uint32_t* mask_src = P.slot_mask + static_cast<size_t>(mask_slot) * W;
  lds_barrier();   // the staged token rows are visible (the Q copies may still be in flight)

  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const int lrow = lane / CH;            // row of each direct load this lane fetches
  const int lch = lane % CH;             // its 16-byte LDS slot in that row
  // Load n fetches rows n*RPI + lrow of a step; lane (lrow, lch) fetches
  // chunk lch ^ kv_swz(R) of row R (LDS slot p of row R holds chunk
  // p ^ kv_swz(R)); one base pointer per load of the wave's share.
  static_assert(NI * RPI == 32 && 32 % kSwzRows<CH> == 0, "the swizzle repeats within a 32-token step");
  const char* lbase[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j)
    lbase[j] = reinterpret_cast<const char*>(kvsel ? vp : kp) + (lch ^ kv_swz<CH>((n0 + j) * RPI + lrow)) * 16;
  // This wave's loads of `step` into ring stage `stage` (staged rows run to a
  // multiple of 512 tokens, entries past the chunk end holding its last
  // token, so a partial last step needs no special case).
  constexpr int OPS_K = NL;                       // vector-memory operations per step
  auto issue = [&](int step, int stage) {
    int32_t rows[NL];
    const int32_t* tr = tok_row + step * 32 + lrow * NI + n0;   // the permuted layout
    if constexpr (NL >= 4) {
#pragma unroll
      for (int j = 0; j < NL; j += 4) {
        const int4 v4 = *reinterpret_cast<const int4*>(tr + j);
        rows[j] = v4.x; rows[j + 1] = v4.y; rows[j + 2] = v4.z; rows[j + 3] = v4.w;
      }
    } else if constexpr (NL == 2) {
      const int2 v2 = *reinterpret_cast<const int2*>(tr);
      rows[0] = v2.x; rows[1] = v2.y;
    } else {
      rows[0] = tr[0];
    }
    const uint32_t sd = ring_lds + stage * STAGE_B;
#pragma unroll
    for (int j = 0; j < NL; ++j)
      lds_dma16(lbase[j] + static_cast<uint64_t>(static_cast<uint32_t>(rows[j])) * ROWB,
                sd + kvsel * TILE_B + (n0 + j) * 1024);
    if (loads_mask) lds_dma4(mask_src + step, sd + 2 * TILE_B + w * 256);
  };
  // waits until at most `later` steps' loads of this wave are outstanding
  auto wait_steps = [&](int later) {
    if (loads_mask) {
      if (later >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * (OPS_K + 1)));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(OPS_K + 1));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    } else {
      if (later >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * OPS_K));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(OPS_K));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
  };
  static_assert(NSTG == 4, "wait_steps covers up to two later steps");

  const int nsteps = (len + 31) / 32;
  // The first NSTG-1 steps go out before the wait for the Q copies, which
  // are older: waiting until only those steps' loads are outstanding covers
  // the copies.
  const int pro = min(NSTG - 1, nsteps);
  for (int s = 0; s < pro; ++s) issue(s, s);
  if (loads_mask) {
    if (pro == 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * (OPS_K + 1)));
    else if (pro == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * (OPS_K + 1)));
    else if (pro == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(OPS_K + 1));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  } else {
    if (pro == 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * OPS_K));
    else if (pro == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * OPS_K));
    else if (pro == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(OPS_K));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
  static_assert(NSTG - 1 == 3, "the prologue waits cover up to three steps");
  lds_barrier();
  // Q^T fragments (B operand of S^T = K Q^T) of this wave's 32 rows: lane
  // (lr, lj) takes d = 32 ks + 8 lj .. +7 of row R = 32w + 16rt + lr, i.e.
  // chunk 4 ks + lj, stored in slot (4 ks + lj) ^ kv_swz(R).
  bf16x8 qf[NRT][KS];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int R = WROWS * w + rt * 16 + lr;
      qf[rt][ks] = *reinterpret_cast<const bf16x8*>(smem + Shape::QOFF + R * ROWB + (((4 * ks + lj) ^ kv_swz<CH>(R)) * 16));
    }

  f32x4 o[DT][NRT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Per row tile: the running max m_run (raw score units) with its exp2
  // offset mc = m_run * scale * log2(e) and rescale threshold thr, both
  // updated only when m_run rises; the lane's true max; and the row sum of
  // P, accumulated by the matrix core against a tile of ones.
  const float cl2 = a.scale_log2;
  float m_run[NRT], m_true[NRT], mc[NRT], thr[NRT];
  f32x4 lacc[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m_run[rt] = kNegInf;
    m_true[rt] = kNegInf;
    mc[rt] = 0.f;
    thr[rt] = kNegInf;
    lacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;

  // LDS byte offsets (within a stage) of this lane's operand fragments: K
  // fragment n = (ks, tt) for S, and the two halves of V^T d-tile dt for PV.
  const int rk0 = 8 * (lr >> 2) + (lr & 3);   // K rows of this lane, per token tile
  int koff[2 * KS], voff[DT][2];
#pragma unroll
  for (int n = 0; n < 2 * KS; ++n) {
    const int ks = n >> 1, R = rk0 + 4 * (n & 1);
    koff[n] = R * ROWB + (((ks * 4 + lj) ^ kv_swz<CH>(R)) * 16);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int R = 8 * lj + 4 * hh + (lr >> 2);
      voff[dt][hh] = TILE_B + R * ROWB + (((2 * dt + ((lr & 3) >> 1)) ^ kv_swz<CH>(R)) * 16) + 8 * (lr & 1);
    }
  const bf16x8 ones8 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f),
                        static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f),
                        static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  // Step i on ring stage STG = i % NSTG (a compile-time constant, so every LDS
  // address is a per-lane base plus an immediate offset).
  auto step_body = [&](auto stg, int i) {
    constexpr int STG = decltype(stg)::value;
    // this wave's loads of step i are done; the barrier makes every wave's
    // visible and tells that every wave has finished step i-1, whose stage
    // is refilled next
    wait_steps(min(NSTG - 2, nsteps - 1 - i));
    lds_barrier();
    if (i + NSTG - 1 < nsteps) issue(i + NSTG - 1, (STG + NSTG - 1) % NSTG);
    if (!active) return;
    const int base = i * 32;
    const char* kb = smem + STG * STAGE_B;
    const uint32_t* mb = reinterpret_cast<const uint32_t*>(kb + 2 * TILE_B);
    bf16x8 kfr[2 * KS];
#pragma unroll
    for (int n = 0; n < 2 * KS; ++n) kfr[n] = *reinterpret_cast<const bf16x8*>(kb + koff[n]);
    __builtin_amdgcn_s_setprio(1);
    f32x4 sacc[2][NRT];
    auto s_tile = [&](auto rtc) {
      constexpr int rt = decltype(rtc)::value;
#pragma unroll
      for (int n = 0; n < 2 * KS; ++n) {
        sacc[n & 1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            kfr[n], qf[rt][n >> 1], n < 2 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[n & 1][rt], 0, 0, 0);
      }
    };
    s_tile(std::integral_constant<int, 0>{});
    // V^T fragments by transpose reads of the token-major V rows (lane (lr,
    // lj) receives V[8lj + 4h' + k][16dt + lr], k = 0..3)
    bf16x8 vfr[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x2 half[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        half[hh] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                       (lds_s16x4_t)(kb + voff[dt][hh])));
      vfr[dt] = __builtin_bit_cast(bf16x8, u32x4{half[0][0], half[0][1], half[1][0], half[1][1]});
    }
    bf16x8 pb[NRT];
    float z[NRT][8];
    const int valid_e = len - base - 8 * lj;   // tokens of this lane's 8 that exist
    const bool all_visible = full && valid_e >= 8;
    auto soft_max = [&](auto rtc) {       // mask, maxima, lazy rescale
      constexpr int rt = decltype(rtc)::value;
      const int rl = WROWS * w + rt * 16 + lr;   // row within the block
      const bool row_ok = rl < nr;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[rt][e] = e < 4 ? sacc[0][rt][e] : sacc[1][rt][e - 4];
      if (!all_visible) {
        const uint32_t bits = row_ok ? (mb[rl] >> (8 * lj)) & 0xffu : 0u;
        // a step of a partly masked chunk whose tokens every row of the tile
        // sees (the prefix part of a chunk that also holds tree tokens) needs
        // no selects
        if (!__all(bits == 0xffu && valid_e >= 8)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) z[rt][e] = (((bits >> e) & 1u) && e < valid_e) ? z[rt][e] : kNegInf;
        }
      } else if (!row_ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) z[rt][e] = kNegInf;
      }
      float mx = z[rt][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[rt][e]);
      m_true[rt] = fmaxf(m_true[rt], mx);
      const bool high = mx > thr[rt];
      if (__any(high)) {
        const float rmx = rowmax4(mx);
        const bool raise = rmx > thr[rt];
        const float mn = raise ? rmx : m_run[rt];
        const float alpha = raise ? fast_exp2((m_run[rt] - mn) * cl2) : 1.f;
        m_run[rt] = mn;
        mc[rt] = mn == kNegInf ? 0.f : mn * cl2;
        thr[rt] = mn + kRescaleSlack / cl2;
        lacc[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
      }
    };
    auto soft_exp = [&](auto rtc) {       // probabilities, bf16 P
      constexpr int rt = decltype(rtc)::value;
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(z[rt][e], cl2, -mc[rt]));   // z = -inf gives 0
      pb[rt] = __builtin_convertvector(p, bf16x8);
    };
    auto pv_tile = [&](auto rtc) {
      constexpr int rt = decltype(rtc)::value;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr[dt], pb[rt], o[dt][rt], 0, 0, 0);
      }
      lacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pb[rt], lacc[rt], 0, 0, 0);
    };
    auto interleave = [] {
#pragma unroll
      for (int k = 0; k < DT; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
    };
    static_assert(NRT == 2 && 2 * KS == DT, "the schedule is written for two row tiles");
    soft_max(std::integral_constant<int, 0>{});
    s_tile(std::integral_constant<int, 1>{});
    soft_exp(std::integral_constant<int, 0>{});
    interleave();
    asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pb[0])));
    soft_max(std::integral_constant<int, 1>{});
    pv_tile(std::integral_constant<int, 0>{});
    soft_exp(std::integral_constant<int, 1>{});
    interleave();
    pv_tile(std::integral_constant<int, 1>{});
    __builtin_amdgcn_s_setprio(0);
  };
  for (int i = 0; i < nsteps; i += NSTG) {
    step_body(std::integral_constant<int, 0>{}, i);
    if (i + 1 < nsteps) step_body(std::integral_constant<int, 1>{}, i + 1);
    if (i + 2 < nsteps) step_body(std::integral_constant<int, 2>{}, i + 2);
    if (i + 3 < nsteps) step_body(std::integral_constant<int, 3>{}, i + 3);
  }

  // The wave's rows are final: M = the row's true max, f = exp2((m_run - M)
  // * scale * log2 e) renormalises l and O to it.  Lane (lr, lj) holds
  // d = 16 dt + 4 lj .. +3 of row 16 rt + lr.
  if (active) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int r = WROWS * w + rt * 16 + lr;
      const float mx = rowmax4(m_true[rt]);
      const float f = (m_run[rt] == kNegInf) ? 0.f : fast_exp2((m_run[rt] - mx) * cl2);
      const float ls = f * lacc[rt][0];
      if (r < nr) {
        const int row = rb + r;
        const int64_t sh = static_cast<int64_t>(gofs + row / a.grp) * a.hq + g * a.grp + row % a.grp;
        if (lj == 0) {
          st_f32<FUSED>(a.pm + sh, mx == kNegInf ? kNegInf : mx * cl2 * kLn2);
          st_f32<FUSED>(a.pl + sh, ls);
        }
        if (a.po_bf16) {
          const float inv = 1.f / lacc[rt][0];    // O / l, independent of the offset
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const f32x4 acc = o[dt][rt];
            const uint32_t lo = pack_bf16x2(acc[0] * inv, acc[1] * inv);
            const uint32_t hi = pack_bf16x2(acc[2] * inv, acc[3] * inv);
            st_u32x2<FUSED>(reinterpret_cast<uint16_t*>(a.po) + sh * D + dt * 16 + lj * 4, lo, hi);
          }
        } else {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) st_f32x4<FUSED>(a.po + sh * D + dt * 16 + lj * 4, f * o[dt][rt]);
        }
      }
    }
  }
  if constexpr (FUSED) {
    fused_publish<ROWS>(P, a.hq, a.grp, rb, nr, gofs, g);
  }
}

// ---------------------------------------------------------------------------
// One launch for all partial work: the plan's wide (128-row) MFMA items take
// the first n_mfma_wide * Hkv work-groups, the 64-row MFMA items the next
// n_mfma * Hkv (dispatched first: the longest), the VALU items the rest, so
// all kinds share the chip instead of running one after the other.  Block b
// of any kind takes KV head b % Hkv (each range is a multiple of Hkv, so a
// head keeps its XCD).  One LDS block serves whichever body the work-group
// runs.
// ---------------------------------------------------------------------------
template <typename T, int D, int R, bool FUSED>
__global__ __launch_bounds__(kPartialThreads) void partial_attention(PartialArgs a) {
  static_assert(64 * valu_waves<R>() == kPartialThreads, "both bodies run 8 waves");
  constexpr int VB = ValuShape<T, D, R>::LDS_B;
  constexpr int MB4 = sizeof(T) == 2 ? MfmaShape<D, 4>::LDS_B : 0;
  constexpr int MB2 = sizeof(T) == 2 ? MfmaShape<D, 2>::LDS_B : 0;
  constexpr int MBG = sizeof(T) == 2 ? MfmaGroupShape<D>::LDS_B : 0;
  constexpr int MB = MB4 > MB2 ? (MB4 > MBG ? MB4 : MBG) : (MB2 > MBG ? MB2 : MBG);
  __shared__ __attribute__((aligned(1024))) char lds[VB > MB ? VB : MB];
  const int ng = a.plan.n_mfma_group * a.hkv;
  const int nw = a.plan.n_mfma_wide * a.hkv;
  const int nm = a.plan.n_mfma * a.hkv;
  const int b = static_cast<int>(blockIdx.x);
  if constexpr (FUSED) {
    const int np = ng + nw + nm + a.plan.n_valu * a.hkv;
    if (b >= np) {
      merge_worker<T, D>(a.merge, a.plan, a.spin_limit, b - np, a.merge_wg_rows);
      return;
    }
  }
  if constexpr (sizeof(T) == 2) {
    if (b < ng) {
      mfma_group_body<D, FUSED>(a, lds, b, 0);
      return;
    }
    if (b < ng + nw) {
      mfma_body<D, FUSED, 2>(a, lds, b - ng, a.plan.n_mfma_group);
      return;
    }
    if (b < ng + nw + nm) {
      mfma_body<D, FUSED, 4>(a, lds, b - ng - nw, a.plan.n_mfma_group + a.plan.n_mfma_wide);
      return;
    }
  }
  valu_body<T, D, R, FUSED>(a, lds, b - ng - nw - nm);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();   // leave no error behind for a later launch check
    return 256;
  }
  return n;
}

// The staging buffer is the source of an asynchronous copy from pageable
// memory; it is rebuilt or freed only after that copy has run.
static hipError_t wait_upload(deft_plan* p) {
  return p->staging_done ? hipEventSynchronize(static_cast<hipEvent_t>(p->staging_done)) : hipSuccess;
}

void release_upload(deft_plan* p) {
  if (!p->staging_done) return;
  (void)wait_upload(p);
  (void)hipEventDestroy(static_cast<hipEvent_t>(p->staging_done));
  p->staging_done = nullptr;
  (void)hipGetLastError();
}

static DevPlan make_dev_plan(const deft_plan* p) {
  const int32_t* b = static_cast<const int32_t*>(p->dev);
  const ImageLayout& L = p->layout;
  DevPlan d;
  d.chunk_start = b + L.chunk_start;
  d.group_offsets = b + L.group_offsets;
  d.chunk_full = b + L.chunk_full;
  d.slot_query = b + L.slot_query;
  d.slot_mask = reinterpret_cast<const uint32_t*>(b + L.slot_mask);
  d.flat_to_logical = b + L.flat_to_logical;
  d.query_slot_offsets = b + L.query_slot_offsets;
  d.query_slots = b + L.query_slots;
  d.mfma_items = reinterpret_cast<const int4*>(b + L.mfma_items);
  d.valu_items = reinterpret_cast<const int4*>(b + L.valu_items);
  d.tickets = const_cast<int32_t*>(b) + L.tickets;
  d.status = const_cast<int32_t*>(b) + L.status;
  d.merge_slots = b + L.merge_slots;
  d.merge_stride = L.merge_stride;
  d.n_mfma_group = L.n_mfma_group;
  d.n_mfma_wide = L.n_mfma_wide;
  d.n_mfma = L.n_mfma;
  d.n_valu = L.n_valu;
  d.mask_words = p->mask_words;
  d.num_queries = p->num_queries;
  return d;
}

// Checks a bounded inter-wave wait makes before it gives up: 2^20 (each
// check sleeps ~64 cycles, so about 30 ms), or DEFT_SPIN_LIMIT from the
// environment when it lies in [0, 2^20] (tests force a give-up with a tiny
// limit).
static int32_t spin_limit() {
  constexpr long kDefault = 1L << 20;
  const char* env = std::getenv("DEFT_SPIN_LIMIT");
  if (env && env[0]) {
    const long v = std::strtol(env, nullptr, 10);
    if (v >= 0 && v <= kDefault) return static_cast<int32_t>(v);
  }
  return static_cast<int32_t>(kDefault);
}

static int hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return DEFT_OK;
  return fail(DEFT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

static bool same_desc(const deft_attn_desc& x, const deft_attn_desc& y) {
  return x.dtype == y.dtype && x.num_q_heads == y.num_q_heads && x.num_kv_heads == y.num_kv_heads &&
         x.head_dim == y.head_dim && x.page_size == y.page_size && x.num_pages == y.num_pages;
}

static int check_ready(const deft_plan* p, const deft_attn_desc* d) {
  if (!p) return fail(DEFT_ERR_INVALID_ARGUMENT, "plan is NULL");
  int rc = check_desc(p, d);
  if (rc) return rc;
  if (!p->uploaded) return fail(DEFT_ERR_INVALID_ARGUMENT, "plan has no device image: call deft_plan_upload");
  if (!same_desc(p->desc, *d))
    return fail(DEFT_ERR_INVALID_ARGUMENT, "desc differs from the desc the plan was uploaded for");
  if (static_cast<int64_t>(d->num_pages) * kPageSize * d->num_kv_heads > INT32_MAX)
    return fail(DEFT_ERR_UNSUPPORTED, "num_pages * page_size * num_kv_heads must fit in int32");
  return DEFT_OK;
}

// Opt-in host check of the block table (environment DEFT_VALIDATE=1): the
// entries of the tree's logical pages are copied back on the stream, which
// is synchronised, and each must lie in [0, num_pages).  Off by default: the
// kernels never range-check block-table entries themselves.
static int validate_block_table(const deft_plan* p, const deft_attn_desc* d, const int32_t* bt,
                                hipStream_t st) {
  const char* env = std::getenv("DEFT_VALIDATE");
  if (!env || env[0] != '1') return DEFT_OK;
  if (!bt) return fail(DEFT_ERR_INVALID_ARGUMENT, "block_table is NULL");
  int32_t last = -1;
  for (int32_t lt : p->flat_to_logical) last = std::max(last, lt);
  const size_t n = static_cast<size_t>(last / kPageSize + 1);
  std::vector<int32_t> h(n);
  hipError_t e = hipMemcpyAsync(h.data(), bt, n * sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_check(e, "DEFT_VALIDATE block-table copy");
  for (size_t i = 0; i < n; ++i)
    if (h[i] < 0 || h[i] >= d->num_pages)
      return fail(DEFT_ERR_INVALID_ARGUMENT, "block_table[" + std::to_string(i) + "] = " + std::to_string(h[i]) +
                                                 " is outside [0, num_pages = " + std::to_string(d->num_pages) + ")");
  return DEFT_OK;
}

template <typename T, int D>
static int launch_partials(const PartialArgs& pa, hipStream_t st) {
  const int hkv = pa.hkv;
  if (sizeof(T) != 2 && pa.plan.n_mfma_group + pa.plan.n_mfma + pa.plan.n_mfma_wide > 0)
    return fail(DEFT_ERR_UNSUPPORTED, "MFMA work for fp32 inputs");
  const int n_partial = (pa.plan.n_mfma_group + pa.plan.n_mfma_wide + pa.plan.n_mfma + pa.plan.n_valu) * hkv;
  if (n_partial == 0) return DEFT_OK;
  // the single-dispatch path appends its merge work-groups
  const int n_merge = pa.fused ? (pa.merge.nq * pa.merge.hq + pa.merge_wg_rows - 1) / pa.merge_wg_rows : 0;
  const dim3 grid(n_partial + n_merge), block(kPartialThreads);
  // the VALU body's row capacity: 4 when every VALU item fits, else 8
  static_assert(kValuRows == 8, "VALU row capacities are 4 and 8");
  const bool r4 = pa.max_valu_rows <= 4;
  if (pa.fused) {
    if (r4) hipLaunchKernelGGL((partial_attention<T, D, 4, true>), grid, block, 0, st, pa);
    else hipLaunchKernelGGL((partial_attention<T, D, 8, true>), grid, block, 0, st, pa);
  } else {
    if (r4) hipLaunchKernelGGL((partial_attention<T, D, 4, false>), grid, block, 0, st, pa);
    else hipLaunchKernelGGL((partial_attention<T, D, 8, false>), grid, block, 0, st, pa);
  }
  return hip_check(hipGetLastError(), "launch of partial_attention");
}

static int run_partials(const void* q, const void* k, const void* v, const int32_t* bt,
                        const deft_plan* p, const deft_attn_desc* d, float* po, float* pm,
                        float* pl, bool po_bf16, hipStream_t st, void* fused_out = nullptr) {
  if (!q || !k || !v || !bt || !po || !pm || !pl)
    return fail(DEFT_ERR_INVALID_ARGUMENT, "device pointers must not be NULL");
  PartialArgs pa;
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.block_table = bt;
  pa.po = po;
  pa.pm = pm;
  pa.pl = pl;
  pa.plan = make_dev_plan(p);
  pa.hq = d->num_q_heads;
  pa.hkv = d->num_kv_heads;
  pa.grp = d->num_q_heads / d->num_kv_heads;
  pa.po_bf16 = po_bf16 ? 1 : 0;
  pa.scale_log2 = kLog2e / std::sqrt(static_cast<float>(d->head_dim));
  pa.spin_limit = spin_limit();
  pa.fused = fused_out != nullptr;
  pa.merge_wg_rows = merge_worker_rows(p->num_queries * d->num_q_heads);
  pa.max_valu_rows = p->layout.max_valu_rows;
  pa.merge.po = po;
  pa.merge.pm = pm;
  pa.merge.pl = pl;
  pa.merge.out = fused_out;
  pa.merge.query_slot_offsets = pa.plan.query_slot_offsets;
  pa.merge.query_slots = pa.plan.query_slots;
  pa.merge.merge_slots = pa.plan.merge_slots;
  pa.merge.merge_stride = pa.plan.merge_stride;
  pa.merge.nq = p->num_queries;
  pa.merge.hq = d->num_q_heads;
  pa.merge.po_bf16 = pa.po_bf16;
  if (d->dtype == DEFT_DTYPE_BF16)
    return d->head_dim == 128 ? launch_partials<uint16_t, 128>(pa, st) : launch_partials<uint16_t, 64>(pa, st);
  return d->head_dim == 128 ? launch_partials<float, 128>(pa, st) : launch_partials<float, 64>(pa, st);
}

static int run_merge(const deft_plan* p, const deft_attn_desc* d, const float* po, const float* pm,
                     const float* pl, void* out, bool po_bf16, hipStream_t st) {
  if (!po || !pm || !pl || !out) return fail(DEFT_ERR_INVALID_ARGUMENT, "device pointers must not be NULL");
  MergeArgs ma;
  ma.po = po;
  ma.pm = pm;
  ma.pl = pl;
  ma.out = out;
  const DevPlan dp = make_dev_plan(p);
  ma.query_slot_offsets = dp.query_slot_offsets;
  ma.query_slots = dp.query_slots;
  ma.merge_slots = dp.merge_slots;
  ma.merge_stride = dp.merge_stride;
  ma.nq = p->num_queries;
  ma.hq = d->num_q_heads;
  ma.po_bf16 = po_bf16 ? 1 : 0;
  const int blocks = (ma.nq * ma.hq + 15) / 16;   // 4 waves of 4 rows
  if (d->dtype == DEFT_DTYPE_BF16) {
    if (d->head_dim == 128) hipLaunchKernelGGL((lse_merge<uint16_t, 128>), dim3(blocks), dim3(256), 0, st, ma);
    else hipLaunchKernelGGL((lse_merge<uint16_t, 64>), dim3(blocks), dim3(256), 0, st, ma);
  } else {
    if (d->head_dim == 128) hipLaunchKernelGGL((lse_merge<float, 128>), dim3(blocks), dim3(256), 0, st, ma);
    else hipLaunchKernelGGL((lse_merge<float, 64>), dim3(blocks), dim3(256), 0, st, ma);
  }
  return hip_check(hipGetLastError(), "launch of lse_merge");
}

// Workspace of deft_tree_attention_noalloc: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  Host code
// never passes `scratch` itself to a kernel (its host-side name is not a
// device address); it looks the device address up once per device with
// hipGetSymbolAddress and passes that pointer.
static_assert(DEFT_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");
static __device__ __align__(256) char scratch[DEFT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;

// Device address of `scratch` on the current device, looked up on the first
// call for that device (with it current) and kept.
static int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxScratchDevices] = {};
  int dev = 0;
  int rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(DEFT_ERR_UNSUPPORTED, "device ordinal " + std::to_string(dev) + " above the no-alloc path's " +
                                          std::to_string(kMaxScratchDevices) + " devices");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    rc = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress of the no-alloc scratch");
    if (rc) return rc;
    if (!p) return fail(DEFT_ERR_HIP, "hipGetSymbolAddress returned NULL for the no-alloc scratch");
    addr[dev] = p;
  }
  *out = addr[dev];
  return DEFT_OK;
}

}  // namespace deft

using deft::fail;

extern "C" {

int deft_plan_upload(deft_plan* p, const deft_attn_desc* d, void* dev_plan, size_t bytes, void* stream) {
  if (!p || !dev_plan) return fail(DEFT_ERR_INVALID_ARGUMENT, "plan and dev_plan must not be NULL");
  if (reinterpret_cast<uintptr_t>(dev_plan) % 256 != 0)
    return fail(DEFT_ERR_INVALID_ARGUMENT, "dev_plan must be 256-byte aligned");
  int rc = deft::hip_check(deft::wait_upload(p), "wait for the previous upload of this plan");
  if (rc) return rc;
  deft::release_upload(p);
  deft::ImageLayout L{};
  rc = deft::build_image(p, d, &p->staging, &L);
  if (rc) return rc;
  if (bytes < 4 * L.total_words) return fail(DEFT_ERR_INVALID_ARGUMENT, "dev_plan buffer too small");
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = deft::hip_check(hipMemcpyAsync(dev_plan, p->staging.data(), 4 * L.total_words,
                                      hipMemcpyHostToDevice, st),
                       "hipMemcpyAsync of the plan image");
  if (rc) return rc;
  // mark the copy's completion on the current device; without an event,
  // finish the copy now
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess && hipEventRecord(e, st) == hipSuccess) {
    p->staging_done = e;
  } else {
    if (e) (void)hipEventDestroy(e);
    (void)hipGetLastError();
    rc = deft::hip_check(hipStreamSynchronize(st), "hipStreamSynchronize after the plan image copy");
    if (rc) return rc;
  }
  p->layout = L;
  p->desc = *d;
  p->dev = dev_plan;
  p->dev_bytes = bytes;
  p->uploaded = true;
  return DEFT_OK;
}

static int check_format(const deft_attn_desc* desc, int32_t fmt) {
  if (fmt == DEFT_PARTIAL_F32) return DEFT_OK;
  if (fmt == DEFT_PARTIAL_BF16_NORM && desc->dtype == DEFT_DTYPE_BF16) return DEFT_OK;
  return fail(DEFT_ERR_INVALID_ARGUMENT, "partial_format must be DEFT_PARTIAL_F32, or DEFT_PARTIAL_BF16_NORM for bf16 inputs");
}

int deft_partial_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const deft_plan* plan,
                           const deft_attn_desc* desc, void* part_o, float* part_m, float* part_l,
                           int32_t partial_format, void* stream) {
  int rc = deft::check_ready(plan, desc);
  if (rc) return rc;
  rc = deft::validate_block_table(plan, desc, block_table, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  rc = check_format(desc, partial_format);
  if (rc) return rc;
  return deft::run_partials(q, k_cache, v_cache, block_table, plan, desc, static_cast<float*>(part_o),
                            part_m, part_l, partial_format == DEFT_PARTIAL_BF16_NORM,
                            static_cast<hipStream_t>(stream));
}

int deft_lse_merge(const deft_plan* plan, const deft_attn_desc* desc, const void* part_o,
                   const float* part_m, const float* part_l, int32_t partial_format, void* out,
                   void* stream) {
  int rc = deft::check_ready(plan, desc);
  if (rc) return rc;
  rc = check_format(desc, partial_format);
  if (rc) return rc;
  return deft::run_merge(plan, desc, static_cast<const float*>(part_o), part_m, part_l, out,
                         partial_format == DEFT_PARTIAL_BF16_NORM, static_cast<hipStream_t>(stream));
}

int deft_tree_attention(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const deft_plan* plan, void* out,
                        const deft_attn_desc* desc, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int rc = deft::check_ready(plan, desc);
  if (rc) return rc;
  rc = deft::validate_block_table(plan, desc, block_table, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  if (!workspace || !out) return fail(DEFT_ERR_INVALID_ARGUMENT, "workspace and out must not be NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(DEFT_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const size_t need = deft::workspace_bytes_for(plan, desc);
  if (workspace_bytes < need) return fail(DEFT_ERR_INVALID_ARGUMENT, "workspace too small");
  // Internal partial format: bf16 O / l for bf16 inputs, fp32 unnormalised O otherwise.
  const bool po_bf16 = deft::bf16_partials(desc);
  const size_t sh = static_cast<size_t>(plan->num_slots) * desc->num_q_heads;
  auto align = [](size_t n) { return (n + 63) & ~static_cast<size_t>(63); };
  float* po = static_cast<float*>(workspace);
  const size_t o_words = deft::partial_o_words(plan, desc);
  float* pm = po + align(o_words);
  float* pl = pm + align(sh);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = deft::run_partials(q, k_cache, v_cache, block_table, plan, desc, po, pm, pl, po_bf16, st);
  if (rc) return rc;
  return deft::run_merge(plan, desc, po, pm, pl, out, po_bf16, st);
}

int deft_tree_attention_fused(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, deft_plan* plan, void* out,
                              const deft_attn_desc* desc, void* workspace, size_t workspace_bytes,
                              void* stream) {
  int rc = deft::check_ready(plan, desc);
  if (rc) return rc;
  rc = deft::validate_block_table(plan, desc, block_table, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  if (!workspace || !out) return fail(DEFT_ERR_INVALID_ARGUMENT, "workspace and out must not be NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(DEFT_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const size_t need = deft::workspace_bytes_for(plan, desc);
  if (workspace_bytes < need) return fail(DEFT_ERR_INVALID_ARGUMENT, "workspace too small");
  const bool po_bf16 = deft::bf16_partials(desc);
  const size_t sh = static_cast<size_t>(plan->num_slots) * desc->num_q_heads;
  auto align = [](size_t n) { return (n + 63) & ~static_cast<size_t>(63); };
  float* po = static_cast<float*>(workspace);
  float* pm = po + align(deft::partial_o_words(plan, desc));
  float* pl = pm + align(sh);
  // One dispatch: partial work-groups, then merge work-groups that wait for
  // their rows' tickets (fused_publish, merge_worker).
  return deft::run_partials(q, k_cache, v_cache, block_table, plan, desc, po, pm, pl, po_bf16,
                            static_cast<hipStream_t>(stream), out);
}

int deft_plan_status(deft_plan* plan, void* stream) {
  if (!plan) return fail(DEFT_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!plan->uploaded) return fail(DEFT_ERR_INVALID_ARGUMENT, "plan has no device image: call deft_plan_upload");
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* word = static_cast<int32_t*>(plan->dev) + plan->layout.status;
  int32_t flag = 0;
  int rc = deft::hip_check(hipMemcpyAsync(&flag, word, sizeof(flag), hipMemcpyDeviceToHost, st),
                           "copy of the plan's status word");
  if (rc) return rc;
  rc = deft::hip_check(hipStreamSynchronize(st), "hipStreamSynchronize for the status word");
  if (rc) return rc;
  if (flag == 0) return DEFT_OK;
  const int32_t zero = 0;
  rc = deft::hip_check(hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, st),
                       "reset of the plan's status word");
  if (rc) return rc;
  rc = deft::hip_check(hipStreamSynchronize(st), "hipStreamSynchronize after the status reset");
  if (rc) return rc;
  return fail(DEFT_ERR_HIP, "a partial-attention work-group ran out of its bounded wait for a partner wave "
                            "(DEFT_SPIN_LIMIT checks); the outputs of the attention calls on this plan since "
                            "the last status check are not valid");
}

int deft_tree_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const deft_plan* plan, void* out,
                                const deft_attn_desc* desc, void* stream) {
  int rc = deft::check_ready(plan, desc);
  if (rc) return rc;
  const size_t need = deft::workspace_bytes_for(plan, desc);
  if (need > DEFT_NOALLOC_SCRATCH_BYTES)
    return fail(DEFT_ERR_UNSUPPORTED, "this plan's partial results need " + std::to_string(need) +
                                          " bytes, above the no-alloc scratch of " +
                                          std::to_string(static_cast<size_t>(DEFT_NOALLOC_SCRATCH_BYTES)) +
                                          " bytes (use deft_tree_attention with a workspace, or a larger "
                                          "chunk_tokens)");
  void* ws = nullptr;
  rc = deft::scratch_address(&ws);
  if (rc) return rc;
  if (!out) return fail(DEFT_ERR_INVALID_ARGUMENT, "out must not be NULL");
  // the same kernels and partial format as deft_tree_attention, on the scratch
  const bool po_bf16 = deft::bf16_partials(desc);
  const size_t sh = static_cast<size_t>(plan->num_slots) * desc->num_q_heads;
  auto align = [](size_t n) { return (n + 63) & ~static_cast<size_t>(63); };
  float* po = static_cast<float*>(ws);
  float* pm = po + align(deft::partial_o_words(plan, desc));
  float* pl = pm + align(sh);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = deft::run_partials(q, k_cache, v_cache, block_table, plan, desc, po, pm, pl, po_bf16, st);
  if (rc) return rc;
  return deft::run_merge(plan, desc, po, pm, pl, out, po_bf16, st);
}

}  // extern "C"
