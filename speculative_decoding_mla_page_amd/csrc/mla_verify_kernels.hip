// gfx950 kernels of tree-masked MLA verify attention: a call is two launches.
//
//   partial_kernel  every workgroup first works out the call's plan from the
//                   serving framework's raw metadata buffers - per-request
//                   lengths and checks, key-range length, the table of
//                   (request, row block, key range) work items ("The
//                   Capture-Safe Kernel", Decisions 1, 2 and 5) - and takes
//                   its own item.  It gathers the item's scattered page_size=1
//                   latent rows through kv_indices / out_cache_loc into LDS
//                   ("The Integration Chasm", The Decision: Adapt the Kernel,
//                   Not the System), builds the tree-visibility words of its
//                   rows from custom_mask, computes S^T = K.Q^T and
//                   O^T += V^T.P^T with bf16 MFMA and fp32 accumulation, keeps
//                   an online softmax per query row, and writes the
//                   unnormalised partial (O, running max, running sum) - the
//                   KV-split partial of the pages' split-K design ("The
//                   Integration Chasm", Context: What Came Before; "The
//                   Capture-Safe Kernel", Decision 3).  A second
//                   instantiation serves compacted pools, taking each prefix
//                   key's slot as the request's first slot + j instead of
//                   reading its index.
//   merge_kernel    combines the partial softmax statistics of each query row
//                   across its key ranges ("The Capture-Safe Kernel", Decision 4)
//                   into the normalised output and its log-sum-exp.
//
// The grids of both depend on the plan only.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "mla_verify_internal.h"

namespace mlav {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// LDS layout of a staged tile of kKeysPerTile keys:
//   V part   : key k's dims [0, 512) at k * 1024 in one of kStages V slots,
//              its 64 16-byte units stored at unit ^ vswz(k);
//   rope part: key k's dims [512, 576) at k * 128 in one of kRopeSlots rope
//              slots (only the score waves read them), units at unit ^ rswz(k).
// Every row is written by one 1 KB direct-to-LDS load (one V row, or the rope
// rows of eight keys), so rows cannot be padded; the swizzles instead spread
// the MFMA operand reads over the banks: the 16 keys of a K-operand read land
// on 16 distinct 16-byte bank groups.
constexpr int kVStride = kDv * 2;                        // 1024 bytes
constexpr int kVSlotBytes = kKeysPerTile * kVStride;     // 32768
constexpr int kRopeSlotBytes = kKeysPerTile * 128;       // 4096
constexpr int kRopeSlots = 3;
__device__ __forceinline__ int vswz(int k) { return k & 15; }
__device__ __forceinline__ int rswz(int k) { return (k >> 1) & 7; }
constexpr int kTilesPerIdx = kIdxKeys / kKeysPerTile;    // 8
constexpr int kRowUnits = kDqk * 2 / 16;   // 16-byte units per latent row
constexpr int kMaxTree = MLA_VERIFY_MAX_TREE_NODES;
constexpr float kRescaleSlack = 8.f;  // rescale O only when a row max grows by > 2^8

// Key order inside a 32-key tile for the PV product.  Lane group g (lanes
// 16g..16g+15) feeds keys kappa(g, 0..7) = {4g..4g+3, 16+4g..16+4g+3} as its
// eight K-dimension slots; these are exactly the keys whose scores the same
// lanes hold in the S^T accumulators (rows 4g+i of each 16-key output tile),
// so P moves from the softmax to the PV operand without any data exchange.

// Row reductions over the four lane groups that hold one query row (lanes
// n, n+16, n+32, n+48): the gfx950 swaps exchange 16-lane rows (xor 16) and
// 32-lane halves (xor 32) in the VALU, with no LDS round trip.
// The larger of two scores as one v_med3_f32: the median of a, b and pinf,
// where pinf holds +inf in a register the compiler cannot see into (with a
// constant +inf the compiler turns the median back into a max).  fmaxf
// costs an extra v_max per operand, because the compiler quiets each input
// first: the hardware max does not follow maxnum for signalling NaNs.
// Scores are finite or -inf; a NaN score only occurs in a poisoned item.
__device__ __forceinline__ float max_sc(float a, float b, float pinf) { return __builtin_amdgcn_fmed3f(a, b, pinf); }
__device__ __forceinline__ float group_max(float v, float pinf) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max_sc(__uint_as_float(a[0]), __uint_as_float(a[1]), pinf);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_sc(__uint_as_float(b[0]), __uint_as_float(b[1]), pinf);
}
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = a[0] | a[1];
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return b[0] | b[1];
}
__device__ __forceinline__ float group_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ int64_t load_index(const void* base, int64_t i, int is64) {
  return is64 ? reinterpret_cast<const int64_t*>(base)[i]
              : static_cast<int64_t>(reinterpret_cast<const int32_t*>(base)[i]);
}

// ceil(a / b) for a >= 0, b >= 1: the 32-bit division when both fit, which
// is several times shorter than the 64-bit one
__device__ __forceinline__ long long div_up(long long a, long long b) {
  if (((unsigned long long)a | (unsigned long long)b) >> 31 == 0) {
    const uint32_t a32 = (uint32_t)a, b32 = (uint32_t)b;
    return (long long)((a32 + b32 - 1) / b32);
  }
  return (a + b - 1) / b;
}

// ---------------------------------------------------------------------------
// the plan of a call, computed on the device from the serving framework's
// raw metadata buffers ("The Capture-Safe Kernel", Decisions 1, 2 and 5):
// every workgroup of the split-partial launch works out the same plan, so no
// launch has to build it first and the grid stays fixed by the host plan
// (Decision 3).
//
// Per request b: T_b = qo_indptr[b+1] - qo_indptr[b], P_b = kv_indptr[b+1] -
// kv_indptr[b] (Decision 2), the checks behind the metadata error bits, and
// its query rows (node, head), heads fastest, cut into 64-row blocks.  Each
// request's combined key range [0, P_b + T_b) is cut into ranges of one
// length shared by all requests, rounded to 32 keys and at least 128.
// Twenty candidate lengths cut the total work W = sum_b rowblocks_b (P_b +
// T_b) into m target_items - f R pieces, for m = 1..4 rounds, R = sum_b
// rowblocks_b and f = 1, 3/4, 1/2, 1/4, 0 (each row block adds at most one
// partly filled range: f = 1 leaves room for all of them, smaller f packs the
// rounds fuller); the one with the least modelled time - rounds of
// target_items workgroups x (tiles per range + the per-item cost, about
// kItemTiles tiles) - among those whose items fit the plan is taken (m = 1,
// f = 0, when none fits: the call is flagged).  Work items are numbered
// request by request, then key range, then row block.
// ---------------------------------------------------------------------------
constexpr int kCands = 20;
// candidate k: the pieces m target_items - f R with m = 1 + k / 5 and
// f = (4 - k % 5) / 4
__device__ __forceinline__ long long cand_slots(int k, int target, int rowblocks) {
  const long long s = (long long)(1 + k / 5) * target - ((long long)rowblocks * (4 - k % 5)) / 4;
  return s < 1 ? 1 : s;
}
constexpr int kFallbackCand = 4;   // m = 1, f = 0: about target_items pieces
constexpr long long kItemTiles = 6;
constexpr int kPlanWaves = kPartialThreads / 64;
struct PlanShared {
  long long w_work[kPlanWaves];        // per-wave partial sums
  int w_rowblocks[kPlanWaves];
  uint32_t w_err[kPlanWaves];
  int w_items[kPlanWaves][kCands];
  int w_scan[kPlanWaves];
  int w_most[kPlanWaves];
  float w_cost[kPlanWaves];            // per wave: its best candidate's modelled time, length, index
  int w_c[kPlanWaves];
  int w_k[kPlanWaves];
  int total_q;
  // the plan
  uint32_t err;
  int chunk;
  int items;
  int max_chunks;
};

template <typename V>
__device__ __forceinline__ V wave_sum(V v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v |= (uint32_t)__shfl_xor((int)v, d);
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d));
  return v;
}

// Reductions over the 64 lanes of a wave, result in every lane: rotations
// inside each 16-lane row (DPP, fused into the add), then the gfx950 row
// swaps across rows.  A few VALU instructions, no LDS round trip.
__device__ __forceinline__ int dpp_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false);   // row_ror:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xf, 0xf, false);   // row_ror:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x122, 0xf, 0xf, false);   // row_ror:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x121, 0xf, 0xf, false);   // row_ror:1
  auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = (int)(a[0] + a[1]);
  auto c = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int)(c[0] + c[1]);
}
__device__ __forceinline__ int dpp_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x122, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x121, 0xf, 0xf, false));
  auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = max((int)a[0], (int)a[1]);
  auto c = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return max((int)c[0], (int)c[1]);
}
__device__ __forceinline__ uint32_t dpp_or(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false);
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = a[0] | a[1];
  auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return c[0] | c[1];
}
// a request's item count under key-range length c, capped so that sums of
// kMaxBatch of them stay in 32 bits (a count that large never fits a plan)
constexpr int kItemsCap = 1 << 20;

// The plan for at most 64 requests (lane b = request b), run by every wave
// of the workgroup on the same inputs: one global round trip for the
// indptrs, then DPP reductions; wave 0 writes the tables.  When the
// candidate lengths have to be timed, the waves share them out and meet at
// one barrier.  The total work is summed in float, which is exact enough to
// pick a range length and, being the same sum in every workgroup, gives
// every workgroup the same plan.
__device__ void plan_call_wave(const KernelParams& p, int32_t (*req)[8], PlanShared& sp) {
  const int lane = threadIdx.x & 63;
  const int wv = (int)(threadIdx.x >> 6);
  const int B = p.batch;
  const int H = p.num_heads;
  const bool full_rows = (p.flags & MLA_VERIFY_FLAG_MASK_FULL_ROWS) != 0;
  const bool have = lane < B;
  int q0 = 0, q1 = 0, k0 = 0, k1 = 0, m0 = 0, m1 = 0;
  if (have) {
    q0 = p.qo_indptr[lane];
    q1 = p.qo_indptr[lane + 1];
    k0 = p.kv_indptr[lane];
    k1 = p.kv_indptr[lane + 1];
    m0 = p.mask_indptr[lane];
    m1 = p.mask_indptr[lane + 1];
  }
  const int T = q1 - q0, P = k1 - k0;
  uint32_t err = 0;
  if (have) {
    if (q0 < 0 || T < 0 || q1 > p.max_q_tokens || (lane == 0 && q0 != 0)) err |= MLA_VERIFY_DEVERR_QO_INDPTR;
    if (k0 < 0 || P < 0 || (long long)k1 > p.max_kv_tokens) err |= MLA_VERIFY_DEVERR_KV_INDPTR;
    if (T > p.max_tree_nodes) err |= MLA_VERIFY_DEVERR_TREE_SIZE;
    const long long mask_size = full_rows ? (long long)T * ((long long)T + P) : (long long)T * T;
    if (m0 < 0 || (long long)(m1 - m0) != mask_size) err |= MLA_VERIFY_DEVERR_MASK_INDPTR;
  }
  const int Tc = T < 0 ? 0 : T, Pc = P < 0 ? 0 : P;
  const int N = Pc + Tc;
  const int rb = (int)(((long long)Tc * H + kRowsPerItem - 1) / kRowsPerItem);
  if (wv == 0 && have) {
    req[lane][RQ_P] = Pc;
    req[lane][RQ_T] = Tc;
    req[lane][RQ_Q0] = q0;
    req[lane][RQ_KV0] = k0;
    req[lane][RQ_RB] = rb;
    req[lane][RQ_MASK0] = m0;
  }
  err = dpp_or(err);
  const int rowblocks = dpp_sum(rb);
  float workf = (float)rb * (float)N;
  workf += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, workf), 0x128, 0xf, 0xf, false));
  workf += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, workf), 0x124, 0xf, 0xf, false));
  workf += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, workf), 0x122, 0xf, 0xf, false));
  workf += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, workf), 0x121, 0xf, 0xf, false));
  workf = group_sum(workf);
  auto items_of = [&](int c) {   // this lane's request under range length c
    return rb > 0 ? (int)min((long long)rb * ((N + c - 1) / c), (long long)kItemsCap) : 0;
  };
  auto cand_len = [&](int k) {   // candidate k's range length
    const float per = ceilf(workf / (float)cand_slots(k, p.target_items, rowblocks));
    const int c = per >= (float)(1 << 30) ? (1 << 30) : ((int)per + kKeysPerTile - 1) / kKeysPerTile * kKeysPerTile;
    return c < kMinChunkKeys ? kMinChunkKeys : c;
  };
  // One round of about target_items ranges (the fallback candidate, the
  // shortest one-round length) is the best plan whenever its items fit in
  // one round: every other one-round candidate is longer, and two rounds cost
  // at least kItemTiles tiles more.  Only otherwise are all candidates timed.
  int chunk_sel = cand_len(kFallbackCand);
  const int items_fb = dpp_sum(items_of(chunk_sel));
  if (items_fb > p.target_items) {   // the same decision in every wave
    // wave w times candidates w, w + kPlanWaves, ...; modelled time: rounds
    // of target_items workgroups x (tiles per range + the per-item cost);
    // float, so that it takes no integer division
    float best = -1.f;
    int best_c = 0, best_k = kCands;
    const float inv_target = 1.f / (float)p.target_items;
    for (int m = wv; m < kCands; m += kPlanWaves) {
      const int c = cand_len(m);
      const int items = dpp_sum(items_of(c));
      const float rounds = fmaxf(1.f, ceilf((float)items * inv_target));
      const float cost = items > p.item_capacity ? -1.f : rounds * (float)(c / kKeysPerTile + kItemTiles);
      if (cost >= 0.f && (best < 0.f || cost < best)) {
        best = cost;
        best_c = c;
        best_k = m;
      }
    }
    if (lane == 0) {
      sp.w_cost[wv] = best;
      sp.w_c[wv] = best_c;
      sp.w_k[wv] = best_k;
    }
    __syncthreads();
    // the least time, the lowest candidate among equals (a serial scan's pick);
    // none fits: the fallback length stays, and the call is flagged below
    best = -1.f;
    best_k = kCands;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
      const float cw = sp.w_cost[w];
      const int kw = sp.w_k[w];
      if (cw >= 0.f && (best < 0.f || cw < best || (cw == best && kw < best_k))) {
        best = cw;
        best_k = kw;
        chunk_sel = sp.w_c[w];
      }
    }
  }
  if (wv != 0) return;   // wave 0 writes the tables
  // each request's first item: an inclusive scan of the item counts over the
  // lanes (DPP: shifts inside each 16-lane row, then the last lane of a row
  // broadcast into the rows after it), less the lane's own count
  const int mine = items_of(chunk_sel);
  int incl = mine;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xf, 0xf, false);   // row_shr:1
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xf, 0xf, false);   // row_shr:2
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xf, 0xf, false);   // row_shr:4
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xf, 0xf, false);   // row_shr:8
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  const int all_items = __builtin_amdgcn_readlane(incl, 63);
  const int chunks = rb > 0 ? (N + chunk_sel - 1) / chunk_sel : 0;
  if (have) {
    req[lane][RQ_CHUNKS] = chunks;
    req[lane][RQ_ITEM0] = incl - mine;
  }
  const int most = dpp_max(chunks);
  const int tq = B > 0 ? __builtin_amdgcn_readlane(q1, B - 1) : 0;
  if (lane == 0) {
    if (all_items > p.item_capacity) err |= MLA_VERIFY_DEVERR_CAPACITY;
    sp.err = err;
    sp.chunk = chunk_sel;
    sp.items = (err & kMetaErrMask) ? 0 : all_items;
    sp.max_chunks = most;
    sp.total_q = tq < 0 ? 0 : (tq > p.max_q_tokens ? p.max_q_tokens : tq);
  }
}

// req: kMaxBatch x 8 int32 of LDS (RQ_* columns).  Up to 64 requests: one
// wave (above).  More: every thread takes requests, one global round trip,
// wave reductions and four barriers.  Ends with a barrier, after which sp's
// plan fields and req hold the plan.
__device__ void plan_call(const KernelParams& p, int32_t (*req)[8], PlanShared& sp) {
  if (p.batch <= 64) {
    plan_call_wave(p, req, sp);
    __syncthreads();
    return;
  }
  constexpr int kThreads = kPartialThreads;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int B = p.batch;
  const int H = p.num_heads;
  const bool full_rows = (p.flags & MLA_VERIFY_FLAG_MASK_FULL_ROWS) != 0;
  uint32_t err = 0;
  long long work = 0;
  int rowblocks = 0;
  if (tid == 0 && B <= 0) sp.total_q = 0;
  for (int b = tid; b < B; b += kThreads) {
    const int q0 = p.qo_indptr[b], q1 = p.qo_indptr[b + 1];
    const int k0 = p.kv_indptr[b], k1 = p.kv_indptr[b + 1];
    const int m0 = p.mask_indptr[b], m1 = p.mask_indptr[b + 1];
    const int T = q1 - q0, P = k1 - k0;
    if (q0 < 0 || T < 0 || q1 > p.max_q_tokens || (b == 0 && q0 != 0)) err |= MLA_VERIFY_DEVERR_QO_INDPTR;
    if (k0 < 0 || P < 0 || (long long)k1 > p.max_kv_tokens) err |= MLA_VERIFY_DEVERR_KV_INDPTR;
    if (T > p.max_tree_nodes) err |= MLA_VERIFY_DEVERR_TREE_SIZE;
    const long long mask_size = full_rows ? (long long)T * ((long long)T + P) : (long long)T * T;
    if (m0 < 0 || (long long)(m1 - m0) != mask_size) err |= MLA_VERIFY_DEVERR_MASK_INDPTR;
    const int Tc = T < 0 ? 0 : T, Pc = P < 0 ? 0 : P;
    const int rb = (Tc * H + kRowsPerItem - 1) / kRowsPerItem;
    req[b][RQ_P] = Pc;
    req[b][RQ_T] = Tc;
    req[b][RQ_Q0] = q0;
    req[b][RQ_KV0] = k0;
    req[b][RQ_RB] = rb;
    req[b][RQ_MASK0] = m0;
    work += (long long)rb * (Pc + Tc);
    rowblocks += rb;
    // query tokens of the call (qo_indptr[B]), clamped to the plan's bound
    if (b == B - 1) sp.total_q = q1 < 0 ? 0 : (q1 > p.max_q_tokens ? p.max_q_tokens : q1);
  }
  work = wave_sum(work);
  rowblocks = wave_sum(rowblocks);
  err = wave_or(err);
  if (lane == 0) {
    sp.w_work[wv] = work;
    sp.w_rowblocks[wv] = rowblocks;
    sp.w_err[wv] = err;
  }
  __syncthreads();
  work = 0;
  rowblocks = 0;
  err = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    work += sp.w_work[w];
    rowblocks += sp.w_rowblocks[w];
    err |= sp.w_err[w];
  }

  // key-range length shared by all requests; every thread works out the
  // candidates (no barrier): they cut the total work into about
  // m x target_items pieces, less the row-block count for m >= 1 (each row
  // block adds at most one partly filled range), rounded up to whole tiles
  auto items_of = [&](int b, int c) {
    const int N = req[b][RQ_P] + req[b][RQ_T];
    const int rb = req[b][RQ_RB];
    return rb > 0 ? rb * ((N + c - 1) / c) : 0;
  };
  int cand[kCands];
#pragma unroll
  for (int m = 0; m < kCands; ++m) {
    const long long slots = cand_slots(m, p.target_items, rowblocks);
    const long long per_item = div_up(work, slots);
    long long c = ((per_item + kKeysPerTile - 1) / kKeysPerTile) * kKeysPerTile;
    if (c < kMinChunkKeys) c = kMinChunkKeys;
    if (c > (1LL << 30)) c = 1LL << 30;
    cand[m] = (int)c;
  }
  {
    int mine[kCands] = {};
    for (int b = tid; b < B; b += kThreads)
#pragma unroll
      for (int m = 0; m < kCands; ++m) mine[m] += items_of(b, cand[m]);
#pragma unroll
    for (int m = 0; m < kCands; ++m) {
      const int t = wave_sum(mine[m]);
      if (lane == 0) sp.w_items[wv][m] = t;
    }
  }
  __syncthreads();
  // the candidate with the least modelled time: rounds of target_items
  // workgroups x (tiles per range + the per-item cost, about kItemTiles
  // tiles), among those whose items fit the plan; none fits: the fallback
  // candidate, flagged
  int chunk_sel = cand[kFallbackCand];
  {
    long long best = -1;
#pragma unroll
    for (int m = 0; m < kCands; ++m) {
      long long items = 0;
#pragma unroll
      for (int w = 0; w < kPlanWaves; ++w) items += sp.w_items[w][m];
      const long long rounds = div_up(items, (long long)p.target_items);
      const long long cost = items > p.item_capacity ? -1 : (rounds < 1 ? 1 : rounds) * (cand[m] / kKeysPerTile + kItemTiles);
      if (cost >= 0 && (best < 0 || cost < best)) {
        best = cost;
        chunk_sel = cand[m];
      }
    }
  }
  // each request's first item: an exclusive scan of the item counts over
  // contiguous runs of requests per thread, inside each wave by shuffles and
  // across the waves through LDS
  const int run = (B + kThreads - 1) / kThreads;
  const int b_lo = min(B, tid * run), b_hi = min(B, b_lo + run);
  int local = 0;
  for (int b = b_lo; b < b_hi; ++b) local += items_of(b, chunk_sel);
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) sp.w_scan[wv] = incl;
  __syncthreads();
  int before = 0, all_items = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int x = sp.w_scan[w];
    before += w < wv ? x : 0;
    all_items += x;
  }
  int most = 0;
  {
    int at = before + incl - local;
    for (int b = b_lo; b < b_hi; ++b) {
      const int N = req[b][RQ_P] + req[b][RQ_T];
      const int rb = req[b][RQ_RB];
      const int chunks = rb > 0 ? (N + chunk_sel - 1) / chunk_sel : 0;
      req[b][RQ_CHUNKS] = chunks;
      req[b][RQ_ITEM0] = at;
      at += items_of(b, chunk_sel);
      most = max(most, chunks);
    }
  }
  most = wave_max(most);
  if (lane == 0) sp.w_most[wv] = most;
  __syncthreads();
  if (tid == 0) {
    int m = 0;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) m = max(m, sp.w_most[w]);
    if (all_items > p.item_capacity) err |= MLA_VERIFY_DEVERR_CAPACITY;
    sp.err = err;
    sp.chunk = chunk_sel;
    sp.items = (err & kMetaErrMask) ? 0 : all_items;
    sp.max_chunks = m;
  }
  __syncthreads();
}

// Last request whose column `col` (a non-decreasing start: RQ_Q0 or
// RQ_ITEM0) is <= x; requests with nothing at x come before the one that
// owns it, so the last one is the owner.
__device__ __forceinline__ int find_request(const int32_t (*req)[8], int B, int col, int x) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (req[mid][col] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// What workgroup 0 of the split-partial launch publishes for the merge and for
// inspection: the header, the request table, and zeroed comparison
// statistics; every workgroup writes the merge's entries of the tokens
// t = blockIdx.x + k * gridDim.x (its request's first token, first item, row
// blocks and key ranges, one 16-byte entry, so the merge searches no table).
__device__ void publish_plan(const KernelParams& p, const int32_t (*req)[8], const PlanShared& sp) {
  const int tid = threadIdx.x;
  const int B = p.batch;
  if (blockIdx.x == 0) {
    for (int b = tid; b < B; b += kPartialThreads) {
      *reinterpret_cast<i32x4*>(p.req + b * 8) = *reinterpret_cast<const i32x4*>(&req[b][0]);
      *reinterpret_cast<i32x4*>(p.req + b * 8 + 4) = *reinterpret_cast<const i32x4*>(&req[b][4]);
    }
    if (tid < (int)(sizeof(mla_verify_compare_stats_t) / 4)) reinterpret_cast<uint32_t*>(p.stats)[tid] = 0;
    if (tid == 0) {
      WsHeader* h = p.hdr;
      h->err = sp.err;
      h->err_meta = sp.err;
      h->n_items = sp.items;
      h->total_q = sp.total_q;
      h->chunk_keys = sp.chunk;
      h->batch = B;
      h->max_chunks = sp.max_chunks;
    }
  }
  const int step = (int)gridDim.x * kPartialThreads;
  for (int t = (int)blockIdx.x + tid * (int)gridDim.x; t < sp.total_q; t += step) {
    const int b = find_request(req, B, RQ_Q0, t);
    *reinterpret_cast<i32x4*>(p.tok + 4 * (size_t)t) =
        i32x4{req[b][RQ_Q0], req[b][RQ_ITEM0], req[b][RQ_RB], req[b][RQ_CHUNKS]};
  }
}

// ---------------------------------------------------------------------------
// split partial: one workgroup of 12 waves per work item (64 query rows x one
// key range), specialised in two roles that run side by side on each SIMD
// (one score wave and two PV waves per SIMD):
//   score waves 0-3: wave r owns query rows 16r..16r+15 (one 16-row MFMA
//     tile); for tile i it forms S^T = K . Q^T, keeps the online softmax of
//     its rows and publishes P(i) = hi + lo and the rows' rescale factors.
//   PV waves 4-11: wave 4+r owns dims [64r, 64r+64) of O for all 64 rows;
//     during tile i it accumulates O^T += V^T . P^T for tile i-1 and moves
//     its eighth of V^T(i) from LDS (transpose load) into registers.
// One barrier per tile (A(i): tile i has landed, P(i-1) is ready); P is
// double buffered.
// ---------------------------------------------------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define MLAV_LDS(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))

// Wait until at most `n` vector-memory operations of this wave are still in
// flight (direct-to-LDS loads complete in issue order and count here), finish
// this wave's LDS operations, then meet the other waves.  The memory clobber
// keeps the compiler from moving LDS accesses across the barrier.  n is one
// of 0, 1, 4 (one tile of 1 or 4 loads).
__device__ __forceinline__ void wait_vm_barrier(int n) {
  if (n >= 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if (n >= 1) asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Direct-to-LDS loads (64 lanes x size bytes to the contiguous LDS bytes at
// M0) written as inline assembly.  Issued through the compiler builtin, a
// later LDS read cannot be told apart from the bytes a load in flight writes,
// and the compiler makes it wait for every load in flight; here every
// consumer waits explicitly instead (wait_vm_barrier), counting on the loads
// of a wave completing in issue order.  The LDS address goes in M0, written
// at least one instruction ahead of the load.
__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)MLAV_LDS(const void, ptr);
}
// row: wave-uniform global address (moved to scalar registers here, so the
// scalar operand holds whatever path computed it); lane_off: this lane's byte
// offset from it
__device__ __forceinline__ void dma16_row(const void* row, uint32_t lane_off, uint32_t lds) {
  const uint64_t a = (uint64_t)(uintptr_t)row;
  const uint64_t sa = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(lane_off), "s"(sa), "{m0}"(lds) : "memory");
}
// addr: this lane's global address
__device__ __forceinline__ void dma16(const void* addr, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(addr), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* addr, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(addr), "{m0}"(lds) : "memory");
}

// A wave-uniform LDS byte offset the compiler cannot see through.  The tile
// loops form their per-iteration LDS addresses from such offsets, so that no
// address becomes an induction register that lives across the whole item:
// such registers get spilled around the item's prologue and reloaded before
// the loop, and the wait for a reload that the compiler places at its first
// use inside the loop waits for every tile load in flight, every iteration.
__device__ __forceinline__ uint32_t opaque_s(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
constexpr int kKRing = 8;                  // K operand reads in flight ahead of the S MFMAs
constexpr int kDvPerWave = kDv / kPVWaves;   // 64 dims of O per PV wave
constexpr int kDtPerWave = kDvPerWave / 16;
static_assert(kRowTiles == 1 && kWaves == 4 && kPVWaves == 8, "four score waves of 16 rows, eight PV waves");
static_assert(kPVWaves * 4 == kKeysPerTile, "each PV wave gathers four keys of a tile");
static_assert(kTilesPerIdx >= 5, "an index block is loaded five tiles ahead of its first use");

// kRowTilesMax: the most 16-row tiles an item of this plan can hold,
// ceil(min(64, max_tree_nodes x H) / 16); an instantiation for fewer than four
// (decode: one node per request) leaves out the PV MFMAs and P reads of row
// tiles that can hold no row.
template <int kRowTilesMax, bool kContig>
__global__ __launch_bounds__(kPartialThreads, 1) void partial_kernel(KernelParams p) {
  __shared__ __attribute__((aligned(128))) unsigned char s_v[kStages * kVSlotBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_r[kRopeSlots * kRopeSlotBytes];
  __shared__ bf16x8 s_p[2][kWaves][2][64];      // P(i) in buffer i & 1: row tile, hi/lo, lane
  __shared__ __attribute__((aligned(16))) uint32_t s_idx[2][kIdxKeys];   // raw slot words of key blocks (double buffered)
  __shared__ f32x4 s_alpha[3][16];              // [i % 3][n][rt]: rescale factor of row 16rt + n
  __shared__ uint32_t s_rescale[3];             // [i % 3]: byte rt != 0 when row tile rt rescaled
  __shared__ uint32_t s_tree_hi[kMaxTree];       // high words of the item's 64-bit tree slots
  __shared__ PlanShared sp;
  static_assert(sizeof(s_v) >= sizeof(int32_t) * kMaxBatch * 8, "the plan tables fit in the V ring");

  const int tid = threadIdx.x;
  const int bid = blockIdx.x;
  const int H = p.num_heads;

  // ---- the call's plan, from the raw metadata; its per-request table lives
  // in the V ring until the first tile loads
  int32_t (*req)[8] = reinterpret_cast<int32_t (*)[8]>(s_v);
  plan_call(p, req, sp);
  publish_plan(p, req, sp);
  // This workgroup's items.  About one workgroup per compute unit, each
  // running its items one after another.  Workgroup g is dispatched to XCD
  // g % 8; XCD x owns the contiguous items [x per, (x + 1) per) (per =
  // ceil(items / 8)), taken by its workgroups in turn, so the row blocks that
  // share a key range (consecutive items) run side by side on one XCD and
  // share its L2.  The plan gives no workgroup more than kMaxItemsPerWg.
  __shared__ int32_t s_mine[kMaxItemsPerWg][12];
  __shared__ int s_nmine;
  {
    const int n_items = sp.items;
    const int g8 = (int)gridDim.x >> 3, x = bid & 7;
    const int per_xcd = (n_items + 7) >> 3;
    const int first = x * per_xcd + (bid >> 3), last = min(n_items, (x + 1) * per_xcd);
    const int count = first < last ? (last - first + g8 - 1) / g8 : 0;
    if (tid < min(count, kMaxItemsPerWg)) {
      const int item = first + tid * g8;
      const int b = find_request(req, p.batch, RQ_ITEM0, item);
      const int rbs = req[b][RQ_RB];
      const int local_item = item - req[b][RQ_ITEM0];
      const int chunk_no = local_item / rbs;
      const int P = req[b][RQ_P], T = req[b][RQ_T];
      const int key0 = chunk_no * sp.chunk;
      int32_t* e = s_mine[tid];
      e[0] = item;
      e[1] = b;
      e[2] = local_item % rbs;
      e[3] = chunk_no;
      e[4] = P;
      e[5] = T;
      e[6] = req[b][RQ_Q0];
      e[7] = req[b][RQ_KV0];
      e[8] = req[b][RQ_MASK0];
      e[9] = key0;
      e[10] = min(P + T, key0 + sp.chunk);
    }
    if (tid == 0) s_nmine = count;
  }
  __syncthreads();   // the plan tables are read
  // (values read from LDS are the same in every lane: readfirstlane keeps
  // them, and everything derived from them, in scalar registers)
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  uint32_t errbits = 0;   // this workgroup's device error bits (thread 0)
  const int n_mine = uni(s_nmine);
  if (n_mine > kMaxItemsPerWg) errbits |= MLA_VERIFY_DEVERR_CAPACITY;
  // The item body, compiled once per role, so that each role's item loop
  // keeps only its own loop-invariant values.
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto run_item = [&](int mi, auto role) {
  constexpr bool kScore = decltype(role)::value;
  // The thread and lane index, formed anew for every item: what the compiler
  // derived from them once, before the item loop, did not stay in registers
  // through it and went to scratch (stores of some 60-96 bytes per lane by
  // every workgroup, about 11 MB of extra HBM writes per launch).
  int tid_item = (int)threadIdx.x;
  asm volatile("" : "+v"(tid_item));
  const int tid = tid_item;
  const int lane = tid & 63;
  const int item = uni(s_mine[mi][0]);
  const int b = uni(s_mine[mi][1]), rb = uni(s_mine[mi][2]), chunk_no = uni(s_mine[mi][3]);
  const int P = uni(s_mine[mi][4]), T = uni(s_mine[mi][5]);
  const int q0 = uni(s_mine[mi][6]), kv0 = uni(s_mine[mi][7]), m0 = uni(s_mine[mi][8]);
  const int key0 = uni(s_mine[mi][9]), key1 = uni(s_mine[mi][10]);
  const int row0 = rb * kRowsPerItem;
  const int nrows = min(kRowsPerItem, T * H - row0);
  if (tid == 0) {
    int32_t* e = p.items + (size_t)item * 8;
    *reinterpret_cast<i32x4*>(e) = i32x4{b, rb, chunk_no, key0};
    *reinterpret_cast<i32x4*>(e + 4) = i32x4{key1, row0, nrows, 0};
  }
  const int ntiles = (key1 - key0 + kKeysPerTile - 1) / kKeysPerTile;
  const int nrt = (nrows + 15) >> 4;            // row tiles with at least one row

  const int r = kScore ? wave : wave - kWaves;   // row tile (score) or dim eighth (PV)
  const int n = lane & 15, g = lane >> 4;
  const int r_local = 16 * r + n;

  // ---- where the keys' slots come from: prefix key j < P from
  // kv_indices[kv0 + j], tree key j >= P from out_cache_loc[q0 + j - P],
  // each int32 or int64 as the plan says.  The tile loop reads the low 32
  // bits of each index (little-endian: the first word of a 64-bit one) and
  // treats a value outside [0, num_slots) as a bad slot: the load reads slot
  // 0 instead and the item is poisoned.  A 64-bit index whose high word is
  // not zero is outside the pool too; the prologue checks those words.
  const bool kv64 = p.kv_idx64 != 0, ocl64 = p.ocl_idx64 != 0;
  const uint32_t nslots = (uint32_t)p.num_slots;
  const int kvw = kv64 ? 8 : 4, oclw = ocl64 ? 8 : 4;
  const unsigned char* kvi = reinterpret_cast<const unsigned char*>(p.kv_indices) + (int64_t)kv0 * kvw;
  // key j >= P's index at ocl_rel + j * oclw
  const unsigned char* ocl_rel =
      reinterpret_cast<const unsigned char*>(p.out_cache_loc) + ((int64_t)q0 - P) * oclw;
  auto idx_ptr = [&](int j) { return j < P ? kvi + (uint32_t)j * kvw : ocl_rel + (uint32_t)j * oclw; };
  auto load_slot = [&](int j) -> uint32_t { return *reinterpret_cast<const uint32_t*>(idx_ptr(j)); };
  // ---- contiguous-prefix fast path (a compacted prefix, "The Integration
  // Chasm", The Decision: Adapt the Kernel, Not the System): prefix key j is
  // slot cb + j with cb = kv_indices[kv0].  The only other prefix indices
  // read are those of the 64-key share that reaches the tree keys (fewer than
  // 64 keys right before them), which a compacted prefix holds as cb + j too.
  // A base outside the pool (or a 64-bit one with a nonzero high word) is
  // replaced by num_slots, so that every prefix key of the request is outside
  // the pool; cb + j stays below 2^32 (both terms are below 2^31).
  // The base is loaded where it is used (the prologues), not kept live
  // through the item.
  const bool contig = kContig && P > 0;
  auto contig_base = [&]() -> uint32_t {
    const uint32_t lo = *reinterpret_cast<const uint32_t*>(kvi);
    const uint32_t hi = kv64 ? *reinterpret_cast<const uint32_t*>(kvi + 4) : 0u;
    return (hi == 0u && lo < nslots) ? lo : nslots;
  };
  uint32_t cb = nslots;   // the score waves' copy, for the slot blocks

  // ---- the fused KV save: with kv_new, every item whose key range holds
  // tree keys first stores its request's draft rows into the pool at
  // out_cache_loc (16 bytes per thread), so its own gathers read them; the
  // items of a request store the same bytes, and the barrier that ends the
  // prologue orders a workgroup's stores before its loads.  Rows whose slot
  // lies outside the pool are not stored (their keys are bad slots).
  if (p.kv_new && key1 > P) {
    const int units = T * kRowUnits;
    for (int u = tid; u < units; u += kPartialThreads) {
      const int t = u / kRowUnits, c = u % kRowUnits;
      const int64_t slot = load_index(p.out_cache_loc, (int64_t)q0 + t, ocl64);
      if (slot < 0 || slot >= p.num_slots) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(p.kv_new + ((int64_t)q0 + t) * p.kv_new_stride_tok + 8 * c);
      *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.kv_pool) + slot * p.kv_row_stride + 8 * c) = v;
    }
  }

  // ---- per-item checks and records (off the tile loop)
  if (p.kv_new && key1 > P) __syncthreads();   // orders the saved rows before this workgroup's gathers
  bool out_of_pool = false;
  bool hidden = false;
  if ((p.flags & MLA_VERIFY_FLAG_CHECK_PREFIX_MASK) && key0 < P) {
    // full-row masks: every prefix column of the range must be nonzero for
    // every node of the request, or the item is poisoned
    const int len = min(key1, P) - key0;
    const int64_t cells = (int64_t)T * len;
    bool h = false;
    for (int64_t c = tid; c < cells; c += kPartialThreads) {
      const int i = (int)(c / len), j = key0 + (int)(c % len);
      h |= p.custom_mask[(int64_t)m0 + (int64_t)i * (P + T) + j] == 0;
    }
    hidden = __syncthreads_or(h);
  }
  if (p.trace && rb == 0) {
    // the gathered slot of every key of the range, as read (computed on the
    // fast path; row block 0's items cover each key once)
    for (int j = key0 + tid; j < key1; j += kPartialThreads) {
      const int64_t raw = j < P ? (contig ? (int64_t)contig_base() + j : load_index(p.kv_indices, (int64_t)kv0 + j, kv64))
                                : load_index(p.out_cache_loc, (int64_t)q0 + (j - P), ocl64);
      p.trace[(int64_t)kv0 + q0 + j] = raw;
    }
  }

  // ---- slot blocks of kIdxKeys keys in LDS (double buffered) ----
  // The score waves copy the raw index words of block b straight into LDS,
  // lane = key, with the tile loads.  Keys past the range end re-read the
  // range's last index.
  // On the fast path a wave whose 64 keys are all prefix keys writes their
  // slot words itself (an LDS store lands no later than the copy would); the
  // one share per request that reaches the tree keys still copies its words.
  auto issue_idx = [&](int blk) {
    const int c0 = key0 + blk * kIdxKeys + 64 * wave;
    const int j = min(c0 + lane, key1 - 1);
    if (contig && min(c0 + 63, key1 - 1) < P) {
      s_idx[blk & 1][64 * wave + lane] = cb + (uint32_t)j;
      return;
    }
    dma4(idx_ptr(j), lds_addr(&s_idx[blk & 1][64 * wave]));
  };
  // ---- direct-to-LDS gather of tile t ----
  // PV wave r fetches the dims [0,512) of keys 4r..4r+3 (one 1 KB load per
  // key, lane = 16-byte unit); score wave w fetches the rope rows of keys
  // 8w..8w+7 (one load).  Keys past the range end re-read the range's last
  // key (finite data, masked).  Loads per tile: 1 (score wave), 4 (PV wave).
  // The slots of a tile are read from LDS one iteration before its loads are
  // issued (read_slots) and used only when they are issued, after the next
  // barrier has waited for every LDS read, so neither the read nor the issue
  // stalls a wave in the middle of its MFMA stream.  Every key of a tile is a
  // V key of exactly one PV wave, which checks it when it issues its load.
  struct TileSlots {
    uint32_t s;   // the raw slot word of this lane's key of a tile: score
                  // waves key 8w + lane / 8 (its rope row), PV waves key
                  // 4r + (lane & 3)
  };
  auto tile_key = [&](int t) {   // this lane's key of tile t, clamped to the range
    const int jt = key0 + t * kKeysPerTile;
    return min(kScore ? jt + 8 * wave + (lane >> 3) : jt + 4 * r + (lane & 3), key1 - 1);
  };
  auto read_slots = [&](int t) {
    const int blk = t / kTilesPerIdx;
    if constexpr (kContig) {
      // A slot block holds a word at every position (keys past the range end
      // repeat the last key's), so a tile key's position needs no clamp; the
      // lane index is formed here, since a lane offset kept from before the
      // loop was spilled around this instantiation's item set-up, and its
      // reload's wait inside the loop would also wait for every tile load in
      // flight.
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const int pos = (t % kTilesPerIdx) * kKeysPerTile + (kScore ? 8 * wave + (ln >> 3) : 4 * r + (ln & 3));
      return TileSlots{s_idx[blk & 1][pos]};
    } else {
      return TileSlots{s_idx[blk & 1][tile_key(t) - (key0 + blk * kIdxKeys)]};
    }
  };
  // the carried slot of a tile key: its pool slot, or kSlotBad outside the pool
  auto carried = [&](uint32_t v) -> int { return v < nslots ? (int)v : kSlotBad; };
  const unsigned char* pool = reinterpret_cast<const unsigned char*>(p.kv_pool);
  const uint32_t row_bytes = (uint32_t)p.kv_row_stride * 2;
  auto row_of = [&](int v) {   // latent row of a carried slot; kSlotBad reads slot 0 (the item is poisoned)
    return pool + (uint64_t)(uint32_t)max(v, 0) * row_bytes;
  };
  // the loads of a tile one at a time, so that the roles can spread them
  // over their MFMA steps
  auto issue_key = [&](int t, const TileSlots& ts, int i) {
    // one key per load: the slot is wave-uniform, so the row address is
    // formed on the scalar unit
    const int kk = 4 * r + i;
    const int v = carried((uint32_t)__builtin_amdgcn_readlane((int)ts.s, i));
    out_of_pool |= v == kSlotBad;
    dma16_row(row_of(v), (uint32_t)(lane ^ vswz(kk)) * 16, lds_addr(s_v + (t % kStages) * kVSlotBytes + kk * kVStride));
  };
  auto issue_rope = [&](int t, const TileSlots& ts) {
    const int kk = 8 * wave + (lane >> 3);
    const int unit = (lane & 7) ^ rswz(kk);
    const int v = carried(ts.s);
    dma16(row_of(v) + 2 * kDv + unit * 16, lds_addr(s_r + (t % kRopeSlots) * kRopeSlotBytes + (8 * wave) * 128));
  };
  auto issue = [&](int t, const TileSlots& ts) {
    if (kScore) {
      issue_rope(t, ts);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) issue_key(t, ts, i);
    }
  };
  const int loads_per_tile = kScore ? 1 : 4;

  // The two roles run separate loops with the same barrier sequence: one
  // barrier A(i) at the top of each iteration i = 0..ntiles.  Iteration i:
  // scores of tile i and P(i) into P buffer i & 1 (score waves) || PV of tile
  // i - 2 from registers, P(i - 1) out of P buffer (i - 1) & 1 and V^T(i)
  // into registers (PV waves); in the last one (i = ntiles) the PV waves also
  // multiply tile ntiles - 1, whose P they have just read.  P(i - 1) is read
  // in iteration i, before the score waves rewrite its buffer in iteration
  // i + 1.  Tile i + 2 goes to the V and rope
  // slots of tile i - 1, free since A(i); its slots were read from LDS in
  // iteration i - 1.
  // Slot block b lands before tile 8b - 5 (issued after tile 8b - 6), and
  // is first read with the slots of tile 8b in iteration 8b - 3; its buffer
  // was last read in iteration 8b - 12.  The waits below count tile loads
  // only: index loads in flight behind a tile make them wait a little longer,
  // never less.
  TileSlots next_slots{};
  // The slots of tiles 0..2 come straight from the index buffers (the same
  // keys, clamped to the range's last one, that the LDS blocks hold), so the
  // first gathers wait for one load instead of the first slot block and a
  // barrier.  The first LDS slot read (tile 3, iteration 0) follows A(0),
  // by which every score wave's first index load has landed.  Loads the
  // compiler issued (queries, these slots) are older than the tile loads, so
  // the tile waits only ever wait longer for them.
  TileSlots pre[3] = {};
  auto load_pre = [&]() {
    const uint32_t cbp = contig ? contig_base() : 0u;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      if (t >= ntiles) break;
      // fast path: a tile of prefix keys only has computed slots
      if (contig && key0 + (t + 1) * kKeysPerTile <= P) pre[t] = TileSlots{cbp + (uint32_t)tile_key(t)};
      else pre[t] = TileSlots{load_slot(tile_key(t))};
    }
  };
  auto prologue = [&]() {
    for (int t = 0; t < 2 && t < ntiles; ++t) issue(t, pre[t]);
    if (2 < ntiles) next_slots = pre[2];
  };
  auto barrier_a = [&](int i) {
    // tile i must have landed; tile i + 1 may still be in flight (the last
    // wait takes everything)
    if (i + 1 < ntiles) wait_vm_barrier(loads_per_tile);
    else wait_vm_barrier(0);
  };
  // what iteration i issues after A(i): tile i + 2, the raw words of slot
  // block i / 8 + 1 (score waves, every 8th iteration) and the slots of tile
  // i + 3
  auto after_a = [&](int i) {
    if (i + 2 < ntiles) issue(i + 2, next_slots);
    if (kScore && i % kTilesPerIdx == 0 && i + kTilesPerIdx < ntiles) issue_idx(i / kTilesPerIdx + 1);
    if (i + 3 < ntiles) next_slots = read_slots(i + 3);
  };


  if constexpr (kScore) {
    // ---- score waves: query rows 16r + n; rows are (node, head), heads fastest
    const bool row_ok = r_local < nrows;
    const bool s_active = r < nrt;
    // the first slot block is on its way while the queries load
    if (contig) cb = contig_base();
    if (ntiles > 0) issue_idx(0);
    // a 64-bit slot must have a zero high word: wave 0 copies those of the
    // item's tree keys (node = lane) into LDS now and checks them after the
    // tile loop, whose waits have seen the copy land
    const bool tree_hi = ocl64 && key1 > P;
    const bool hi_lane = wave == 0 && P + lane >= key0 && P + lane < key1;
    if (tree_hi && wave == 0 && hi_lane) dma4(ocl_rel + (uint32_t)(P + lane) * 8 + 4, lds_addr(&s_tree_hi[0]));
    load_pre();
    bf16x8 qf[kDqk / 32];
    uint64_t anc = 0;
    {
      const int rr = row0 + r_local;
      const int node = rr / H, head = rr % H;
      const int tok = q0 + node;
      const uint16_t* qrow = p.q + (int64_t)tok * p.q_stride_tok + (int64_t)head * p.q_stride_head;
#pragma unroll
      for (int ks = 0; ks < kDqk / 32; ++ks) {
        u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(qrow + ks * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
      if (key1 > P) {
        // tree word of the row's node ("The Capture-Safe Kernel", Decision
        // 5): bit k = its custom_mask entry for tree node k (T x T blocks, or
        // the tree columns of full rows).  Lane group g reads entries
        // 16g..16g+15 of the row; the four groups' pieces are joined across
        // lanes.
        // The sixteen byte loads are unconditional, so that they are all in
        // flight together (a load under a lane condition got a branch and a
        // wait of its own each): a row past the item's rows reads node 0's
        // entries and an entry past T reads entry T - 1, both in the block,
        // and the conditions are applied to the loaded bytes.
        const bool full = (p.flags & MLA_VERIFY_FLAG_MASK_FULL_ROWS) != 0;
        const int node_c = row_ok ? node : 0;
        const uint8_t* mrow = p.custom_mask + (int64_t)m0 + (full ? P : 0) + (int64_t)node_c * (full ? P + T : T);
        uint8_t mb[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) mb[k] = mrow[min(16 * g + k, T - 1)];
        uint32_t bits = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int kk = 16 * g + k;
          if (row_ok && kk < T && mb[k] != 0) bits |= 1u << k;
        }
        const uint32_t lo = group_or(g == 0 ? bits : g == 1 ? bits << 16 : 0u);
        const uint32_t hi = group_or(g == 2 ? bits : g == 3 ? bits << 16 : 0u);
        anc = ((uint64_t)hi << 32) | lo;
        // recorded once per node (its head-0 row) for inspection
        if (g == 0 && row_ok && head == 0) p.anc[tok] = anc;
      }
    }
    float m_run = -INFINITY, l_run = 0.f;       // softmax state of this lane's row
    float m_use = 0.f;                           // m_run, or 0 while it is -inf
    float pinf = INFINITY;                       // for max_sc
    asm volatile("" : "+s"(pinf));
    //   K for S^T (A operand): key 16kt + n, unit 4ks + g (ks < 16) ->
    //   k_lo[ks & 3] + 256 (ks >> 2) + 16 kt * 1024; rope unit 4(ks - 16) + g.
    //   The swizzle only touches the low 4 bits of a unit index, so the rest
    //   of every address is an instruction immediate.
    int k_lo[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) k_lo[kq] = n * kVStride + (((4 * kq + g) ^ vswz(n)) << 4);
    const int r_off = n * 128 + ((g ^ rswz(n)) * 16);          // ks = 16
    const int r_off2 = n * 128 + (((4 + g) ^ rswz(n)) * 16);   // ks = 17

    // row tiles without rows contribute P = 0 and never rescale
#pragma unroll
    for (int bf = 0; bf < 2; ++bf) {
      s_p[bf][r][0][lane] = bf16x8{};
      s_p[bf][r][1][lane] = bf16x8{};
    }
    if (lane == 0)
#pragma unroll
      for (int bf = 0; bf < 3; ++bf) reinterpret_cast<uint8_t*>(&s_rescale[bf])[r] = 0;
    // the query loads are waited for here, before the first gathers: left
    // to the compiler, that wait sat inside the tile loop, where on the
    // hardware it also waits for every tile load in flight
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) asm volatile("" :: "v"(qf[ks]));
    prologue();

    for (int i = 0; i <= ntiles; ++i) {
      barrier_a(i);
      if (!s_active || i >= ntiles) {
        after_a(i);
        continue;
      }
      const bool more = i + 2 < ntiles;
      const unsigned char* vslot = s_v + opaque_s((uint32_t)(i % kStages) * kVSlotBytes);
      const unsigned char* rslot = s_r + opaque_s((uint32_t)(i % kRopeSlots) * kRopeSlotBytes);
      const int jt = key0 + i * kKeysPerTile;
      // S^T = K . Q^T: 32 keys x 16 rows, K-dim 576.  The two 16-key halves
      // alternate, so the two independent accumulator chains can issue back
      // to back; operand reads run kKRing steps ahead of the MFMAs
      constexpr int kSSteps = 2 * (kDqk / 32);
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      auto k_operand = [&](int step) -> bf16x8 {
        const int kt = step & 1, ks = step >> 1;
        const unsigned char* ap = ks < 16 ? vslot + k_lo[ks & 3] + (ks >> 2) * 256 + 16 * kt * kVStride
                                          : rslot + 16 * kt * 128 + (ks == 16 ? r_off : r_off2);
        return *reinterpret_cast<const bf16x8*>(ap);
      };
      // the scores gate the next PV step: the score wave goes ahead of the PV
      // waves on its SIMD for the S MFMAs; during its softmax the PV waves
      // (priority 1) go first and fill the MFMA pipe
      __builtin_amdgcn_s_setprio(3);
      bf16x8 ka[kKRing];
#pragma unroll
      for (int s = 0; s < kKRing; ++s) ka[s] = k_operand(s);
#pragma unroll
      for (int step = 0; step < kSSteps; ++step) {
        const int kt = step & 1, ks = step >> 1;
        const bf16x8 a = ka[step % kKRing];
        if (step + kKRing < kSSteps) ka[step % kKRing] = k_operand(step + kKRing);
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], sacc[kt], 0, 0, 0);
        // the tile loads of this iteration ride along with the MFMAs
        if (step == 2 && more) issue_rope(i + 2, next_slots);
        if (step == 6 && i % kTilesPerIdx == 0 && i + kTilesPerIdx < ntiles) issue_idx(i / kTilesPerIdx + 1);
        if (step == 8 && i + 3 < ntiles) next_slots = read_slots(i + 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // mask the range tail and invisible tree keys (raw scores: the scale,
      // positive, is applied to the row max and inside the exponent)
      const bool need_mask = jt + kKeysPerTile > min(P, key1);
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = jt + 16 * kt + 4 * g + q;
            bool vis = j < key1;
            if (j >= P) vis = vis && ((anc >> (j - P)) & 1ull);
            sacc[kt][q] = vis ? sacc[kt][q] : -INFINITY;
          }
        }
      }
      // the tile max in base-2 units: scaling by a positive factor commutes
      // with the max, rounding included
      float mx = max_sc(max_sc(max_sc(sacc[0][0], sacc[0][1], pinf), max_sc(sacc[0][2], sacc[0][3], pinf), pinf),
                        max_sc(max_sc(sacc[1][0], sacc[1][1], pinf), max_sc(sacc[1][2], sacc[1][3], pinf), pinf),
                        pinf);
      mx = group_max(mx, pinf) * p.sm_scale_log2;
      // lazy rescale: move a row's reference max only when the tile max
      // exceeds it by more than 2^kRescaleSlack (then p <= 2^8 stays safe)
      const bool need = mx > m_run + kRescaleSlack;
      const bool any_need = __builtin_amdgcn_ballot_w64(need) != 0;
      float alpha = 1.f;
      if (any_need) {
        // a branch, not selects: the compiler would otherwise compute this
        // rare path on every tile
        asm volatile("");
        const float m_new = need ? mx : m_run;
        alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
        m_use = m_run == -INFINITY ? 0.f : m_run;
      }
      // p = 2^(scale s - m) and its split into bf16 hi + lo: hi = p rounded
      // to bf16, lo = p - hi (exact in fp32) rounded to bf16, so hi + lo
      // carries p to about 2^-17.  Pairs are converted together, and hi is
      // widened back from the packed pair.
      float pv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) pv[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[k >> 2][k & 3], p.sm_scale_log2, -m_use));
      const float rs = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
      u32x4 hi4, lo4;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x2 hp = {(__bf16)pv[2 * k], (__bf16)pv[2 * k + 1]};
        uint32_t hb = __builtin_bit_cast(uint32_t, hp);
        // the widened halves come from the packed pair (otherwise the
        // compiler converted the low element a second time)
        asm volatile("" : "+v"(hb));
        hi4[k] = hb;
        const float l0 = pv[2 * k] - __builtin_bit_cast(float, hb << 16);
        const float l1 = pv[2 * k + 1] - __builtin_bit_cast(float, hb & 0xffff0000u);
        const bf16x2 lp = {(__bf16)l0, (__bf16)l1};
        lo4[k] = __builtin_bit_cast(uint32_t, lp);
      }
      l_run += group_sum(rs);
      s_p[i & 1][r][0][lane] = __builtin_bit_cast(bf16x8, hi4);
      s_p[i & 1][r][1][lane] = __builtin_bit_cast(bf16x8, lo4);
      // the rescale flags and factors of tile i, read by the PV waves in
      // iterations i + 1 and i + 2 (triple buffered: rewritten in i + 3)
      if (any_need && g == 0)
        *reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(&s_alpha[0][n]) + 4 * r +
                                  opaque_s((uint32_t)(i % 3) * sizeof(s_alpha[0]))) = alpha;
      if (lane == 0) reinterpret_cast<uint8_t*>(&s_rescale[i % 3])[r] = any_need;
    }
    if (tree_hi && hi_lane) out_of_pool |= s_tree_hi[lane] != 0u;
    if (kv64 && !contig) {
      // the high words of the range's 64-bit prefix indices
      for (int j = key0 + tid; j < min(key1, P); j += kWaves * 64)
        out_of_pool |= *reinterpret_cast<const uint32_t*>(kvi + (uint32_t)j * 8 + 4) != 0u;
    }
    // a poisoned item (a slot outside the pool, or a prefix key a checked
    // full-row mask hides) gives its rows m = +inf, l = NaN; its bits go to this
    // workgroup's error slot, which the merge launch folds into the header
    out_of_pool = __syncthreads_or(out_of_pool);
    const bool poison = out_of_pool || hidden;
    if (tid == 0)
      errbits |= (out_of_pool ? (uint32_t)MLA_VERIFY_DEVERR_SLOT_RANGE : 0u) |
                 (hidden ? (uint32_t)MLA_VERIFY_DEVERR_MASK_PREFIX : 0u);
    if (row_ok && g == 0) {
      float* pm = p.part_ml + ((size_t)item * kRowsPerItem + r_local) * 2;
      // a poisoned item: m = +inf, l = NaN (the merge then gives NaN rows
      // even when none of the item's scores was finite)
      pm[0] = poison ? INFINITY : m_run;
      pm[1] = poison ? NAN : l_run;
    }
  } else {
    // ---- PV waves: O for all 64 rows, dims [64r, 64r + 64); o[dt][rt]
    // holds, in lane (g, n), O[row 16rt + n][dim 64r + 16dt + 4g + i]
    f32x4 o[kDtPerWave][kWaves];
#pragma unroll
    for (int dt = 0; dt < kDtPerWave; ++dt)
#pragma unroll
      for (int rt = 0; rt < kWaves; ++rt) o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    //   V^T (A operand, transposed read): lane s = 4k + j of group g points at
    //   key 4g + k (and 16 + 4g + k), dims 64r + 16dt + 4j, i.e. unit
    //   8r + 2dt + (j >> 1), byte 8 (j & 1)
    //   The unit index is (8r + h) + 2dt where 8r + h has bits 1-2 clear, so
    //   the swizzled unit of dim tile dt is that of dim tile 0 with 2dt
    //   xored in: dim tile dt sits at byte v_lo0 ^ (dt << 5) of the slot.  The
    //   slots start at multiples of 128 bytes, so the xor can be applied to
    //   the whole LDS address of the current slot; one register holds the
    //   offsets of all four dim tiles.
    int v_lo0;
    {
      const int v_key = 4 * g + (n >> 2);
      v_lo0 = v_key * kVStride + (n & 1) * 8 + ((((kDvPerWave / 8) * r + ((n >> 1) & 1)) ^ vswz(v_key)) << 4);
    }
    static_assert(kDvPerWave / 8 == 8 && kDtPerWave == 4 && kVSlotBytes % 128 == 0,
                  "dim tile dt only flips bits 5-6 of the byte offset");
    load_pre();
    prologue();
    // The PV waves run two tiles behind the score waves: iteration i
    // multiplies tile i - 2 with operands that are all in registers by then
    // (P(i - 2) and its rescale flags, read in iteration i - 1; V^T(i - 2),
    // read in iteration i - 2), and meanwhile reads P(i - 1) and V^T(i).  A
    // row tile's rescale factors are read from LDS only when its flag is set
    // (rarely), so no register holds them.
    // vt[s][dt] is the A operand for dims 64r + 16dt, keys kappa(g, 0..7), of
    // the tile with parity s.
    bf16x8 vt[2][kDtPerWave];
    bf16x8 ph[kWaves], pl[kWaves];
    uint32_t resc = 0;   // rescale flags of the tile read last (wave-uniform: a scalar register)
    auto v_operand = [&](const unsigned char* vslot, int dt) -> bf16x8 {
      const uint32_t vb = (lds_addr(vslot) + (uint32_t)v_lo0) ^ (uint32_t)(dt << 5);
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)vb);
      const i16x4 vc = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vb + 16 * kVStride));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vc, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto read_p = [&](int t, int rt) {   // P(t) of row tile rt
      ph[rt] = s_p[t & 1][rt][0][lane];
      pl[rt] = s_p[t & 1][rt][1][lane];
    };

    // one iteration; the parity of i is a compile-time constant so that the
    // two V^T register sets are addressed statically
    // PV of the last tile, in the iteration that reads its P (ntiles): its
    // V^T is in register set sv ^ 1 (read in the iteration before), its P and
    // rescale flags were loaded in this iteration.  No iteration follows
    // only to drain the two-tile lag.
    auto final_pv = [&](auto parity) {
      constexpr int sv = decltype(parity)::value;
      const int ab = (ntiles - 1) % 3;
#pragma unroll
      for (int rt = 0; rt < kWaves; ++rt) {
        if (rt < kRowTilesMax) {
          if ((resc >> (8 * rt)) & 0xffu) {
            const float alpha = s_alpha[ab][n][rt];
#pragma unroll
            for (int dt = 0; dt < kDtPerWave; ++dt) o[dt][rt] *= alpha;
          }
#pragma unroll
          for (int dt = 0; dt < kDtPerWave; ++dt)
            o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[sv ^ 1][dt], ph[rt], o[dt][rt], 0, 0, 0);
#pragma unroll
          for (int dt = 0; dt < kDtPerWave; ++dt)
            o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[sv ^ 1][dt], pl[rt], o[dt][rt], 0, 0, 0);
        }
      }
    };
    __builtin_amdgcn_s_setprio(1);
    auto pv_iteration = [&](int i, auto parity) {
      constexpr int sv = decltype(parity)::value;   // = i & 1: V^T(i - 2) in, V^T(i) out
      barrier_a(i);
      const unsigned char* vslot = s_v + opaque_s((uint32_t)(i % kStages) * kVSlotBytes);
      const bool v_next = i < ntiles;              // V^T(i) to read
      const bool p_next = i >= 1 && i <= ntiles;   // P(i - 1) to read
      if (i < 2) {
        if (v_next) {
#pragma unroll
          for (int dt = 0; dt < kDtPerWave; ++dt) vt[sv][dt] = v_operand(vslot, dt);
        }
        if (p_next) {
          resc = uni(s_rescale[(i - 1) % 3]);
#pragma unroll
          for (int rt = 0; rt < kWaves; ++rt) read_p(i - 1, rt);
        }
        after_a(i);
        if (i == ntiles && ntiles > 0) final_pv(parity);
        return;
      }
      const bool more_dma = i + 2 < ntiles;
      const bool more_slots = i + 3 < ntiles;
      const uint32_t resc_cur = resc;
      const int ab = (i - 2) % 3;                  // tile i - 2's factors
      if (p_next) resc = uni(s_rescale[(i - 1) % 3]);
      // PV of tile i - 2, one row tile at a time (row tiles without rows
      // carry P = 0, so there are no branches but the rare rescale; row tiles
      // past kRowTilesMax are left out at compile time); each P operand, once
      // used, is replaced by P(i - 1), and in the last pass each V^T operand
      // by V^T(i)
#pragma unroll
      for (int rt = 0; rt < kWaves; ++rt) {
        if (rt < kRowTilesMax) {
          if ((resc_cur >> (8 * rt)) & 0xffu) {
            const float alpha = s_alpha[ab][n][rt];
#pragma unroll
            for (int dt = 0; dt < kDtPerWave; ++dt) o[dt][rt] *= alpha;
          }
#pragma unroll
          for (int dt = 0; dt < kDtPerWave; ++dt)
            o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[sv][dt], ph[rt], o[dt][rt], 0, 0, 0);
#pragma unroll
          for (int dt = 0; dt < kDtPerWave; ++dt) {
            o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[sv][dt], pl[rt], o[dt][rt], 0, 0, 0);
            if (rt == kWaves - 1 && v_next) vt[sv][dt] = v_operand(vslot, dt);
          }
          if (p_next) read_p(i - 1, rt);
        } else if (rt == kWaves - 1 && v_next) {
#pragma unroll
          for (int dt = 0; dt < kDtPerWave; ++dt) vt[sv][dt] = v_operand(vslot, dt);
        }
        // the tile loads of this iteration ride along with the MFMAs, right
        // after the first row tile's, so their issue stalls come early
        if (rt == 0 && more_dma) {
#pragma unroll
          for (int k = 0; k < 4; ++k) issue_key(i + 2, next_slots, k);
        }
        if (rt == 2 && more_slots) next_slots = read_slots(i + 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i == ntiles) final_pv(parity);
    };
    for (int i = 0; i <= ntiles; i += 2) {
      pv_iteration(i, std::integral_constant<int, 0>{});
      if (i + 1 <= ntiles) pv_iteration(i + 1, std::integral_constant<int, 1>{});
    }
    // the partial O does not depend on the poison flags (a poisoned item's l
    // is NaN): store it before the flag reductions
#pragma unroll
    for (int rt = 0; rt < kWaves; ++rt) {
      const int rl = 16 * rt + n;
      if (rl >= nrows) continue;
      float* po = p.part_o + ((size_t)item * kRowsPerItem + rl) * kDv + kDvPerWave * r;
#pragma unroll
      for (int dt = 0; dt < kDtPerWave; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g) = o[dt][rt];
    }
    out_of_pool = __syncthreads_or(out_of_pool);
  }
  };
  const int n_run = min(n_mine, kMaxItemsPerWg);
  if (wave < kWaves) {
    for (int mi = 0; mi < n_run; ++mi) run_item(mi, std::true_type{});
  } else {
    for (int mi = 0; mi < n_run; ++mi) run_item(mi, std::false_type{});
  }
  if (tid == 0) p.errs[bid] = (int32_t)errbits;
}

// ---------------------------------------------------------------------------
// merge ("The Capture-Safe Kernel", Decision 4): each partial carries (O, m, l)
// relative to its own reference max m (base-2 units); with m* = max_c m_c a
// query row (token, head) is sum_c 2^(m_c - m*) O_c / sum_c 2^(m_c - m*) l_c
// and lse = (m* + log2 L) ln 2.  A row with no visible key: out = 0,
// lse = -inf.
// A workgroup of eight waves takes 8 / w consecutive rows, w waves per row,
// where w (1, 2, 4 or 8) is the fewest waves that cover the longest
// request's key ranges kMergeUnroll at a time.  Wave s of a row takes its
// ranges c = s, s + w, ... (lane = 8 of the 512 dims), kMergeUnroll per pass
// with all their loads in flight, and folds them into a running (m, l, O);
// the w wave results are combined the same way through LDS.  A row waits for
// two memory round trips: the header together with the token entries of the
// four possible row mappings, then the partials.  Workgroups past the last
// row exit at once.
// Besides, workgroup 0 folds the split-partial workgroups' error slots into
// the header's error word.
// ---------------------------------------------------------------------------
constexpr int kMergeUnroll = 8;
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(KernelParams p) {
  constexpr int kMW = kMergeThreads / 64;
  __shared__ f32x4 s_acc[kMW][2][64];
  __shared__ float s_m[kMW], s_l[kMW];
  __shared__ uint32_t s_err;
  const WsHeader* hdr = p.hdr;
  const int H = p.num_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t err = hdr->err_meta;
  const int total_q = hdr->total_q;
  const int most = hdr->max_chunks;
  // the token entry of this wave's row under each mapping w = 1, 2, 4, 8,
  // loaded beside the header (clamped to the region; used only when live)
  i32x4 tk_w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row_k = (int)blockIdx.x * (kMW >> k) + (wave >> k);
    const int t_k = min(row_k / H, p.max_q_tokens - 1);
    tk_w[k] = *reinterpret_cast<const i32x4*>(p.tok + 4 * (size_t)t_k);
  }
  if (blockIdx.x == 0) {
    // every device error bit of the call: the metadata checks and each
    // split-partial workgroup's slot
    if (tid == 0) s_err = err;
    __syncthreads();
    uint32_t e = 0;
    for (int w = tid; w < p.partial_grid; w += kMergeThreads) e |= (uint32_t)p.errs[w];
    if (e) atomicOr(&s_err, e);
    __syncthreads();
    if (tid == 0) p.hdr->err = s_err;
  }
  int lw = 0, wpr = 1;   // waves per row = 2^lw
  while (wpr < kMW && wpr * kMergeUnroll < most) {
    wpr <<= 1;
    ++lw;
  }
  const int rows_per_wg = kMW / wpr;
  const int row = blockIdx.x * rows_per_wg + wave / wpr;
  const int sub = wave % wpr;
  const int t = row / H, h = row % H;
  if (blockIdx.x * rows_per_wg >= total_q * H) return;   // the whole workgroup is past the last row
  // a row past the last one does no work but still meets the barrier below
  const bool live = t < total_q;
  float* outp = p.out + (int64_t)t * p.out_stride_tok + (int64_t)h * p.out_stride_head;
  float* lsep = p.lse ? p.lse + (int64_t)t * p.lse_stride_tok + h : nullptr;
  if (err & kMetaErrMask) {
    if (live && sub == 0) {
      *reinterpret_cast<f32x4*>(outp + 8 * lane) = f32x4{NAN, NAN, NAN, NAN};
      *reinterpret_cast<f32x4*>(outp + 8 * lane + 4) = f32x4{NAN, NAN, NAN, NAN};
      if (lsep && lane == 0) *lsep = NAN;
    }
    return;
  }
  const i32x4 tk = live ? tk_w[lw] : i32x4{0, 0, 0, 0};   // q0, item0, row blocks, chunks
  const int r = (t - tk[0]) * H + h;
  const int rb = r / kRowsPerItem, lr = r % kRowsPerItem;
  const int item0 = tk[1], rbs = tk[2], chunks = live ? tk[3] : 0;
  auto item_of = [&](int c) { return (size_t)(item0 + c * rbs + rb) * kRowsPerItem + lr; };

  // fold weights 2^(m_c - M) into a running (M, L, acc); a range with no
  // visible key (m_c = -inf) adds nothing.  A poisoned range carries m_c =
  // +inf and l_c = NaN: it takes the running max to +inf, its weight is
  // 2^(inf - inf) = NaN, and every later rescale is NaN too, so the row
  // comes out NaN.
  float M = -INFINITY, L = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = sub; c0 < chunks; c0 += wpr * kMergeUnroll) {
    float m[kMergeUnroll], l[kMergeUnroll];
    f32x4 v[kMergeUnroll][2];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int c = c0 + u * wpr;
      m[u] = -INFINITY;
      l[u] = 0.f;
      v[u][0] = v[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c < chunks) {
        const size_t ix = item_of(c);
        m[u] = p.part_ml[ix * 2];
        l[u] = p.part_ml[ix * 2 + 1];
        const float* po = p.part_o + ix * kDv + 8 * lane;
        v[u][0] = *reinterpret_cast<const f32x4*>(po);
        v[u][1] = *reinterpret_cast<const f32x4*>(po + 4);
      }
    }
    float mg = M;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) mg = fmaxf(mg, m[u]);
    if (mg == -INFINITY) continue;
    const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mg);
    L *= sc;
    acc0 *= sc;
    acc1 *= sc;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float w = m[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[u] - mg);
      L += w * l[u];
      acc0 += w * v[u][0];
      acc1 += w * v[u][1];
    }
    M = mg;
  }
  if (wpr > 1) {
    // the row's other waves hand their (M, L, acc) to its first wave
    if (sub > 0) {
      s_acc[wave][0][lane] = acc0;
      s_acc[wave][1][lane] = acc1;
      if (lane == 0) {
        s_m[wave] = M;
        s_l[wave] = L;
      }
    }
    __syncthreads();
    if (sub > 0 || !live) return;
    float mstar = M;
    for (int w = 1; w < wpr; ++w) mstar = fmaxf(mstar, s_m[wave + w]);
    if (mstar != -INFINITY) {
      const float s0 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mstar);
      L *= s0;
      acc0 *= s0;
      acc1 *= s0;
      for (int w = 1; w < wpr; ++w) {
        const float mw = s_m[wave + w];
        const float sw = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mstar);
        L += sw * s_l[wave + w];
        acc0 += sw * s_acc[wave + w][0][lane];
        acc1 += sw * s_acc[wave + w][1][lane];
      }
    }
    M = mstar;
  }
  if (!live) return;
  f32x4 r0, r1;
  float lse;
  if (M == -INFINITY) {
    r0 = r1 = f32x4{0.f, 0.f, 0.f, 0.f};
    lse = -INFINITY;
  } else {
    const float inv = 1.f / L;
    r0 = acc0 * inv;
    r1 = acc1 * inv;
    lse = (M + __builtin_amdgcn_logf(L)) * 0.69314718055994531f;
  }
  *reinterpret_cast<f32x4*>(outp + 8 * lane) = r0;
  *reinterpret_cast<f32x4*>(outp + 8 * lane + 4) = r1;
  if (lsep && lane == 0) *lsep = lse;
}

// ---------------------------------------------------------------------------
constexpr int kCompareThreads = 128;
__device__ __forceinline__ float bf16_ulp_at(float r) {
  // 2^(floor(log2 |r|) - 7) with |r| floored at 2^-126
  const uint32_t e = (__float_as_uint(r) >> 23) & 0xffu;   // biased exponent
  const uint32_t ee = e < 1u ? 1u : e;                      // zero and subnormals: as 2^-126
  // 2^(ee - 134): normal for ee >= 8, else the subnormal with that one bit set
  return __uint_as_float(ee >= 8u ? (ee - 7u) << 23 : 1u << (15u + ee));
}
__global__ __launch_bounds__(kCompareThreads) void compare_kernel(KernelParams p) {
  __shared__ uint32_t s_max, s_over, s_nan;
  const int H = p.num_heads;
  const int row = blockIdx.x;
  const int t = row / H, h = row % H;
  if (t >= p.hdr->total_q) return;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_max = 0;
    s_over = 0;
    s_nan = 0;
  }
  __syncthreads();
  const f32x4 o = *reinterpret_cast<const f32x4*>(p.out + (int64_t)t * p.out_stride_tok +
                                                  (int64_t)h * p.out_stride_head + 4 * tid);
  const f32x4 r = *reinterpret_cast<const f32x4*>(p.ref_out + (int64_t)t * p.ref_out_stride_tok +
                                                  (int64_t)h * p.ref_out_stride_head + 4 * tid);
  uint32_t mx = 0, over = 0, nan = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool on = isnan(o[k]), rn = isnan(r[k]);
    if (on != rn) {
      ++nan;
      ++over;
    } else if (!on) {
      const float d = fabsf(o[k] - r[k]);
      if (isfinite(d)) mx = max(mx, __float_as_uint(d));
      if (!(d <= 2.f * bf16_ulp_at(r[k])) && o[k] != r[k]) ++over;
    }
  }
  atomicMax(&s_max, mx);
  if (over) atomicAdd(&s_over, over);
  if (nan) atomicAdd(&s_nan, nan);
  __syncthreads();
  if (tid == 0) {
    mla_verify_compare_stats_t* st = p.stats;
    atomicMax(&st->max_abs_diff_bits, s_max);
    if (s_over) atomicAdd(&st->count_over, s_over);
    if (s_nan) atomicAdd(&st->count_nan_mismatch, s_nan);
    atomicAdd(&st->count_total, (uint32_t)kDv);
    if (p.ref_lse && p.lse) {
      const float a = p.lse[(int64_t)t * p.lse_stride_tok + h];
      const float b = p.ref_lse[(int64_t)t * p.ref_lse_stride_tok + h];
      if (isfinite(a) && isfinite(b)) atomicMax(&st->max_lse_diff_bits, __float_as_uint(fabsf(a - b)));
      else if (isfinite(a) != isfinite(b) || isnan(a) != isnan(b)) atomicAdd(&st->count_lse_mismatch, 1u);
    }
  }
}

int launch_compare(const KernelParams& p, const mla_verify_layout_t& lay, void* stream) {
  if (lay.merge_grid <= 0) return 0;
  hipLaunchKernelGGL(compare_kernel, dim3(lay.merge_grid), dim3(kCompareThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// prefix compaction: one wave per prefix row (grid-stride over all rows of
// the batch).  The wave reads the row's old slot, copies its 72 16-byte units
// (lanes 0-63, then lanes 0-7 again), then lane 0 rewrites the index, so every
// read of the old index precedes its rewrite.
// ---------------------------------------------------------------------------
constexpr int kCompactThreads = 256;
constexpr int kCompactGroups = 1024;
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(KernelParams p, const int64_t* dst_start,
                                                                  int32_t* error_word) {
  __shared__ int s_k0[kMaxBatch + 1];
  const int B = p.batch;
  if (B <= 0) return;
  const int kB = p.kv_indptr[B];
  if (kB < 0 || (int64_t)kB > p.max_kv_tokens) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(error_word, (int32_t)MLA_VERIFY_DEVERR_KV_INDPTR);
    return;
  }
  for (int b = threadIdx.x; b <= B; b += kCompactThreads) s_k0[b] = p.kv_indptr[b];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * (kCompactThreads / 64);
  uint16_t* pool = const_cast<uint16_t*>(p.kv_pool);
  for (int g = blockIdx.x * (kCompactThreads / 64) + (int)(threadIdx.x >> 6); g < kB; g += waves) {
    int lo = 0, hi = B - 1;   // last request whose prefix starts at or before g
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_k0[mid] <= g) lo = mid; else hi = mid - 1;
    }
    const int k0 = s_k0[lo], k1 = s_k0[lo + 1];
    if (k0 < 0 || k1 < k0 || g >= k1) {
      if (lane == 0) atomicOr(error_word, (int32_t)MLA_VERIFY_DEVERR_KV_INDPTR);
      continue;
    }
    const int64_t src = load_index(p.kv_indices, g, p.kv_idx64);
    const int64_t dst = dst_start[lo] + (g - k0);
    if (src < 0 || src >= p.num_slots || dst < 0 || dst >= p.num_slots) {
      if (lane == 0) atomicOr(error_word, (int32_t)MLA_VERIFY_DEVERR_SLOT_RANGE);
      continue;
    }
    const uint16_t* from = pool + src * p.kv_row_stride;
    uint16_t* to = pool + dst * p.kv_row_stride;
    const u32x4 a = *reinterpret_cast<const u32x4*>(from + 8 * lane);
    u32x4 b2 = u32x4{0u, 0u, 0u, 0u};
    if (lane < kRowUnits - 64) b2 = *reinterpret_cast<const u32x4*>(from + 8 * (64 + lane));
    *reinterpret_cast<u32x4*>(to + 8 * lane) = a;
    if (lane < kRowUnits - 64) *reinterpret_cast<u32x4*>(to + 8 * (64 + lane)) = b2;
    if (lane == 0) {
      if (p.kv_idx64) reinterpret_cast<int64_t*>(const_cast<void*>(p.kv_indices))[g] = dst;
      else reinterpret_cast<int32_t*>(const_cast<void*>(p.kv_indices))[g] = (int32_t)dst;
    }
  }
}

int launch_compact(const KernelParams& p, const int64_t* dst_start, int32_t* error_word, void* stream) {
  // one wave per row, up to kCompactGroups workgroups of 4 waves
  int64_t groups = (p.max_kv_tokens + kCompactThreads / 64 - 1) / (kCompactThreads / 64);
  if (groups > kCompactGroups) groups = kCompactGroups;
  if (groups < 1) groups = 1;
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)groups), dim3(kCompactThreads), 0, (hipStream_t)stream, p,
                     dst_start, error_word);
  return (int)hipGetLastError();
}

template <bool kContig>
static void launch_partial_tiles(const KernelParams& p, const mla_verify_layout_t& lay, int tiles, void* stream) {
  if (tiles <= 1)
    hipLaunchKernelGGL((partial_kernel<1, kContig>), dim3(lay.partial_grid), dim3(kPartialThreads), 0,
                       (hipStream_t)stream, p);
  else if (tiles == 2)
    hipLaunchKernelGGL((partial_kernel<2, kContig>), dim3(lay.partial_grid), dim3(kPartialThreads), 0,
                       (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((partial_kernel<kWaves, kContig>), dim3(lay.partial_grid), dim3(kPartialThreads), 0,
                       (hipStream_t)stream, p);
}

int launch_partial(const KernelParams& p, const mla_verify_layout_t& lay, void* stream) {
  // the most rows an item of this plan holds bound its 16-row tiles; the
  // contiguous-prefix fast path is an instantiation of its own, so that the
  // index path's code is unchanged by it
  const int64_t rows = (int64_t)p.max_tree_nodes * p.num_heads;
  const int tiles = rows >= kRowsPerItem ? kWaves : (int)((rows + 15) / 16);
  if (p.flags & MLA_VERIFY_FLAG_CONTIGUOUS_PREFIX) launch_partial_tiles<true>(p, lay, tiles, stream);
  else launch_partial_tiles<false>(p, lay, tiles, stream);
  return (int)hipGetLastError();
}

int launch_merge(const KernelParams& p, const mla_verify_layout_t& lay, void* stream) {
  if (lay.merge_grid <= 0) return 0;
  hipLaunchKernelGGL(merge_kernel, dim3(lay.merge_grid), dim3(kMergeThreads), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace mlav
