// gfx950 kernels of tree-masked MLA verify attention.
//
//   meta_kernel     per-request lengths and validation, packed tree-visibility
//                   words, and the table of (request, row block, key range)
//                   work items, all derived on the device from the serving
//                   framework's raw metadata buffers ("The Capture-Safe Kernel",
//                   Decisions 1, 2 and 5).
//   partial_kernel  one workgroup per work item: gathers the item's scattered
//                   page_size=1 latent rows through kv_indices / out_cache_loc
//                   into LDS ("The Integration Chasm", The Decision: Adapt the
//                   Kernel, Not the System), computes S^T = K.Q^T and
//                   O^T += V^T.P^T with bf16 MFMA and fp32 accumulation, keeps
//                   an online softmax per query row, and writes the unnormalised
//                   partial (O, running max, running sum) - the KV-split partial
//                   of the pages' split-K design ("The Integration Chasm",
//                   Context: What Came Before; "The Capture-Safe Kernel",
//                   Decision 3).
//   merge_kernel    combines the partial softmax statistics of each query row
//                   across its key ranges ("The Capture-Safe Kernel", Decision 4)
//                   into the normalised output and its log-sum-exp.
//
// The grids of all three depend on the plan only.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "mla_verify_internal.h"

namespace mlav {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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
constexpr float kRescaleSlack = 8.f;  // rescale O only when a row max grows by > 2^8

// Key order inside a 32-key tile for the PV product.  Lane group g (lanes
// 16g..16g+15) feeds keys kappa(g, 0..7) = {4g..4g+3, 16+4g..16+4g+3} as its
// eight K-dimension slots; these are exactly the keys whose scores the same
// lanes hold in the S^T accumulators (rows 4g+i of each 16-key output tile),
// so P moves from the softmax to the PV operand without any data exchange.

__device__ __forceinline__ int64_t load_index(const void* base, int64_t i, int is64) {
  return is64 ? reinterpret_cast<const int64_t*>(base)[i]
              : static_cast<int64_t>(reinterpret_cast<const int32_t*>(base)[i]);
}

// ---------------------------------------------------------------------------
// slot staging (metadata launch, workgroups 1..): every request's keys in
// combined order (prefix keys from kv_indices, then its tree nodes' own keys
// from out_cache_loc), at kv_indptr[b] + qo_indptr[b] + j, as int32 pool
// slots, -1 for a slot outside [0, num_slots).  The split-partial kernel then
// reads one contiguous, checked int32 list per request.  A request whose
// indptrs are out of range is skipped (workgroup 0 flags it and plans no
// work); every read stays inside the ranges the indptrs were checked against.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// metadata launch, workgroups 1..: per-key and per-token staging beside the
// planning in workgroup 0.  Each group takes a contiguous share of the keys
// and every groups-th token, and reads the index buffers within the ranges
// the indptrs were checked against; a request whose indptrs or mask size are
// out of range is skipped (workgroup 0 flags it and plans no work).
//
//   slots: every request's keys in combined order (prefix keys from
//     kv_indices, then its tree nodes' own keys from out_cache_loc), at
//     kv_indptr[b] + qo_indptr[b] + j, as int32 pool slots; -1 for a slot
//     outside [0, num_slots), -2 for a prefix key whose full-row mask column
//     hides it from some node (with the prefix check).  The split-partial
//     kernel reads one contiguous, checked list per request.
//   tree words: bit k of token t's word is its mask entry for tree node k of
//     its request (T x T blocks, or full rows of P + T entries whose tree part
//     starts at column P); one wave per token, lane k reads entry k and a
//     ballot packs the row.
//   fused KV save: draft token t's latent row kv_new[t] goes to pool slot
//     out_cache_loc[t], 16 bytes per thread (72 per row), before the partial
//     launch gathers it; slots outside the pool are not stored.
// The loads of one pass are all issued before the first of them is used, so
// a group waits for about two memory round trips.
// ---------------------------------------------------------------------------
constexpr int kRowUnits = kDqk * 2 / 16;   // 16-byte units per latent row
__device__ void meta_staging(const KernelParams& p, int group, int groups) {
  const int B = p.batch;
  if (B <= 0) return;
  // per request, in LDS: where its keys start, its prefix start and length,
  // its first query token and key count (0 for a request whose indptrs are
  // out of range)
  __shared__ int s_start[kMaxBatch], s_k0[kMaxBatch], s_P[kMaxBatch], s_q0[kMaxBatch], s_N[kMaxBatch];
  __shared__ int s_m0[kMaxBatch];   // full-row mask block of the request, -1 when not checked
  __shared__ int s_tm0[kMaxBatch];  // tree columns of its node 0's mask row, -1 when unreadable
  __shared__ int s_qB, s_kB;
  const bool check_prefix = (p.flags & MLA_VERIFY_FLAG_CHECK_PREFIX_MASK) != 0;
  const bool full_rows = (p.flags & MLA_VERIFY_FLAG_MASK_FULL_ROWS) != 0;
  if (threadIdx.x == 0) {
    s_qB = p.qo_indptr[B];
    s_kB = p.kv_indptr[B];
  }
  for (int b = threadIdx.x; b < B; b += kMetaThreads) {
    const int q0 = p.qo_indptr[b], q1 = p.qo_indptr[b + 1];
    const int k0 = p.kv_indptr[b], k1 = p.kv_indptr[b + 1];
    const int m0 = p.mask_indptr[b], m1 = p.mask_indptr[b + 1];
    const bool ok = q0 >= 0 && q1 >= q0 && q1 <= p.max_q_tokens && k0 >= 0 && k1 >= k0 &&
                    (int64_t)k1 <= p.max_kv_tokens;
    s_start[b] = k0 + q0;
    s_k0[b] = k0;
    s_P[b] = k1 - k0;
    s_q0[b] = q0;
    s_N[b] = ok ? (k1 - k0) + (q1 - q0) : 0;
    // mask rows are read only where the block has the size its layout gives
    const long long T = q1 - q0;
    const long long sq = T * T, full = T * ((long long)(k1 - k0) + T);
    const bool m_ok = ok && m0 >= 0 && (long long)m1 - m0 == (full_rows ? full : sq);
    s_m0[b] = (check_prefix && full_rows && m_ok) ? m0 : -1;
    s_tm0[b] = (m_ok && T <= p.max_tree_nodes && T <= 64) ? m0 + (full_rows ? k1 - k0 : 0) : -1;
  }
  __syncthreads();
  const int qB = s_qB, kB = s_kB;
  if (qB < 0 || qB > p.max_q_tokens || kB < 0 || (int64_t)kB > p.max_kv_tokens) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kW = kMetaThreads / 64;

  // tree word of token t: where this lane's mask entry is, -1 when it has none
  // (also for a whole row that is not read)
  auto tree_entry = [&](int t) -> long long {
    int lo = 0, hi = B - 1;   // last request whose tokens start at or before t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_q0[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int m0 = s_tm0[lo];
    const int T = s_N[lo] - s_P[lo];
    const int i = t - s_q0[lo];
    if (m0 < 0 || i < 0 || i >= T || lane >= T) return -1;
    return (long long)m0 + (long long)i * (full_rows ? s_P[lo] + T : T) + lane;
  };
  auto tree_row_valid = [&](int t) {
    // the row is written when its request's mask is readable (lane 0 always
    // has an entry then, T >= 1)
    return __builtin_amdgcn_readfirstlane((int)(tree_entry(t) >= 0 ? 1 : 0));
  };
  // this wave's first token: its entry is loaded now and packed after the
  // slot loads below have been issued
  const int t_first = group * kW + wave;
  const long long e_first = t_first < qB ? tree_entry(t_first) : -1;
  const int row_first = t_first < qB ? tree_row_valid(t_first) : 0;
  const uint8_t m_first = e_first >= 0 ? p.custom_mask[e_first] : 0;

  // fused KV save: this thread's first unit of the new rows (the rest below)
  const int64_t units = p.kv_new ? (int64_t)qB * kRowUnits : 0;
  const int64_t u_first = (int64_t)group * kMetaThreads + threadIdx.x;
  u32x4 sv = u32x4{0u, 0u, 0u, 0u};
  int64_t sslot = -1;
  if (u_first < units) {
    const int t = (int)(u_first / kRowUnits), c = (int)(u_first % kRowUnits);
    sv = *reinterpret_cast<const u32x4*>(p.kv_new + (int64_t)t * p.kv_new_stride_tok + 8 * c);
    sslot = load_index(p.out_cache_loc, t, p.ocl_idx64);
  }

  const int total = qB + kB;
  const int per = (total + groups - 1) / groups;
  const int g0 = group * per, g1 = min(total, g0 + per);
  // kPer positions per thread at a time: every index load is issued before
  // the first store.  A thread's positions only grow, so the request that
  // holds one (the last request whose keys start at or before it) is found
  // by walking forward from the one that held the previous position; the
  // walk starts at the request of the group's first position.
  constexpr int kPer = 8;
  int lo = 0;
  {
    int hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= g0) lo = mid; else hi = mid - 1;
    }
  }
  int r_start = s_start[lo], r_next = lo + 1 < B ? s_start[lo + 1] : INT_MAX;
  for (int base = g0; base < g1; base += kPer * kMetaThreads) {
    int64_t raw[kPer];
    bool have[kPer], hidden[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int g = base + k * kMetaThreads + (int)threadIdx.x;
      have[k] = false;
      hidden[k] = false;
      raw[k] = 0;
      if (g >= g1) continue;
      while (g >= r_next) {
        ++lo;
        r_start = r_next;
        r_next = lo + 1 < B ? s_start[lo + 1] : INT_MAX;
      }
      const int j = g - r_start;
      if (j < 0 || j >= s_N[lo]) continue;
      const int P = s_P[lo];
      raw[k] = j < P ? load_index(p.kv_indices, (int64_t)s_k0[lo] + j, p.kv_idx64)
                     : load_index(p.out_cache_loc, (int64_t)s_q0[lo] + (j - P), p.ocl_idx64);
      have[k] = true;
      if (j < P && s_m0[lo] >= 0) {
        // column j of every node's full mask row must be nonzero
        const int T = s_N[lo] - P;
        const uint8_t* col = p.custom_mask + s_m0[lo] + j;
        for (int i = 0; i < T; ++i) hidden[k] |= col[(size_t)i * (P + T)] == 0;
      }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      if (!have[k]) continue;
      const int g = base + k * kMetaThreads + (int)threadIdx.x;
      p.slots[g] = hidden[k] ? kSlotMaskedPrefix : (raw[k] >= 0 && raw[k] < p.num_slots) ? (int32_t)raw[k] : -1;
      if (p.trace) p.trace[g] = raw[k];
    }
  }

  {
    const uint64_t w = __builtin_amdgcn_ballot_w64(m_first != 0);
    if (row_first && lane == 0) p.anc[t_first] = w;
  }
  for (int t = t_first + groups * kW; t < qB; t += groups * kW) {
    const long long e = tree_entry(t);
    const int row = tree_row_valid(t);
    const bool vis = e >= 0 && p.custom_mask[e] != 0;
    const uint64_t w = __builtin_amdgcn_ballot_w64(vis);
    if (row && lane == 0) p.anc[t] = w;
  }

  uint16_t* pool = const_cast<uint16_t*>(p.kv_pool);
  for (int64_t u = u_first; u < units; u += (int64_t)groups * kMetaThreads) {
    if (u != u_first) {
      const int t = (int)(u / kRowUnits), c = (int)(u % kRowUnits);
      sv = *reinterpret_cast<const u32x4*>(p.kv_new + (int64_t)t * p.kv_new_stride_tok + 8 * c);
      sslot = load_index(p.out_cache_loc, t, p.ocl_idx64);
    }
    if (sslot < 0 || sslot >= p.num_slots) continue;
    *reinterpret_cast<u32x4*>(pool + sslot * p.kv_row_stride + 8 * (int)(u % kRowUnits)) = sv;
  }
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
// metadata build: workgroup 0 (the slot staging runs beside it)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMetaThreads) void meta_kernel(KernelParams p) {
  if (blockIdx.x > 0) {
    meta_staging(p, blockIdx.x - 1, gridDim.x - 1);
    return;
  }
  __shared__ int32_t s_req[kMaxBatch][8];
  __shared__ uint32_t s_err;
  __shared__ long long s_work;
  __shared__ int s_rowblocks;
  constexpr int kCands = 5;
  __shared__ int s_scan[kMetaThreads / 64];
  __shared__ int s_cand[kCands];
  __shared__ int s_cand_items[kCands];
  __shared__ long long s_cand_cost[kCands];
  __shared__ int32_t s_chunk;
  __shared__ int32_t s_items;
  __shared__ int32_t s_total_q;
  __shared__ int32_t s_max_chunks;
  const int tid = threadIdx.x;
  const int B = p.batch;
  const int H = p.num_heads;
  if (tid == 0) {
    s_err = 0;
    s_work = 0;
    s_rowblocks = 0;
    s_items = 0;
    s_max_chunks = 0;
    for (int m = 0; m < kCands; ++m) s_cand_items[m] = 0;
  }
  __syncthreads();
  if (tid == 0) {
    // query tokens of the call, clamped to the plan's bound
    int tq = B > 0 ? p.qo_indptr[B] : 0;
    s_total_q = tq < 0 ? 0 : (tq > p.max_q_tokens ? p.max_q_tokens : tq);
  }

  // per-request lengths and checks (prefix length = kv_indptr[b+1] - kv_indptr[b])
  const bool full_rows = (p.flags & MLA_VERIFY_FLAG_MASK_FULL_ROWS) != 0;
  if (tid < (int)(sizeof(mla_verify_compare_stats_t) / 4)) reinterpret_cast<uint32_t*>(p.stats)[tid] = 0;
  uint32_t err = 0;
  long long work = 0;
  int rowblocks = 0;
  for (int b = tid; b < B; b += kMetaThreads) {
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
    const int rows = Tc * H;
    const int rb = (rows + kRowsPerItem - 1) / kRowsPerItem;
    s_req[b][RQ_P] = Pc;
    s_req[b][RQ_T] = Tc;
    s_req[b][RQ_Q0] = q0;
    s_req[b][RQ_KV0] = k0;
    s_req[b][RQ_RB] = rb;
    s_req[b][RQ_MASK0] = m0;
    work += (long long)rb * (Pc + Tc);
    rowblocks += rb;
  }
  if (err) atomicOr(&s_err, err);
  if (work) atomicAdd(reinterpret_cast<unsigned long long*>(&s_work), (unsigned long long)work);
  if (rowblocks) atomicAdd(&s_rowblocks, rowblocks);
  __syncthreads();

  // key-range length shared by all requests.  Candidates cut the total (row
  // block x key) work into about m x target_items pieces (less the row-block
  // count, since every row block adds at most one partly filled range),
  // rounded up to whole tiles; the one chosen has the least modelled time:
  // rounds of target_items workgroups x (tiles per range + the per-item
  // cost, about kItemTiles tiles), among those whose items fit the plan.
  // Thread m works out candidate m, so the 64-bit divisions run side by side.
  auto items_of = [&](int b, int c) {
    const int N = s_req[b][RQ_P] + s_req[b][RQ_T];
    const int rb = s_req[b][RQ_RB];
    return rb > 0 ? rb * ((N + c - 1) / c) : 0;
  };
  constexpr long long kItemTiles = 6;
  if (tid < kCands) {
    long long slots = tid == 0 ? (long long)p.target_items : (long long)tid * p.target_items - s_rowblocks;
    if (slots < 1) slots = 1;
    const long long per_item = div_up(s_work, slots);
    long long c = ((per_item + kKeysPerTile - 1) / kKeysPerTile) * kKeysPerTile;
    if (c < kMinChunkKeys) c = kMinChunkKeys;
    if (c > (1LL << 30)) c = 1LL << 30;
    s_cand[tid] = (int)c;
  }
  __syncthreads();
  int cand[kCands];
#pragma unroll
  for (int m = 0; m < kCands; ++m) cand[m] = s_cand[m];
  {
    int mine[kCands] = {0, 0, 0, 0, 0};
    for (int b = tid; b < B; b += kMetaThreads)
#pragma unroll
      for (int m = 0; m < kCands; ++m) mine[m] += items_of(b, cand[m]);
#pragma unroll
    for (int m = 0; m < kCands; ++m)
      if (mine[m]) atomicAdd(&s_cand_items[m], mine[m]);   // zeroed at the start
  }
  __syncthreads();
  if (tid < kCands) {
    // modelled cost of candidate m, -1 when its items do not fit
    const long long items = s_cand_items[tid];
    const long long rounds = div_up(items, (long long)p.target_items);
    s_cand_cost[tid] = items > p.item_capacity ? -1 : (rounds < 1 ? 1 : rounds) * (cand[tid] / kKeysPerTile + kItemTiles);
  }
  __syncthreads();
  // the first candidate of least cost; none fits: cand[0], flagged below
  int chunk_sel = cand[0];
  {
    long long best = -1;
#pragma unroll
    for (int m = 0; m < kCands; ++m) {
      const long long cost = s_cand_cost[m];
      if (cost >= 0 && (best < 0 || cost < best)) {
        best = cost;
        chunk_sel = cand[m];
      }
    }
  }
  // each request's first item: an exclusive scan of the item counts over
  // contiguous runs of requests per thread, inside each wave by shuffles and
  // across the waves through LDS
  const int run = (B + kMetaThreads - 1) / kMetaThreads;
  const int b_lo = min(B, tid * run), b_hi = min(B, b_lo + run);
  int local = 0;
  for (int b = b_lo; b < b_hi; ++b) local += items_of(b, chunk_sel);
  const int lane = tid & 63, wv = tid >> 6;
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_scan[wv] = incl;
  __syncthreads();
  int before = 0, all_items = 0;
#pragma unroll
  for (int w = 0; w < kMetaThreads / 64; ++w) {
    const int x = s_scan[w];
    before += w < wv ? x : 0;
    all_items += x;
  }
  {
    int at = before + incl - local;
    int most = 0;
    for (int b = b_lo; b < b_hi; ++b) {
      const int N = s_req[b][RQ_P] + s_req[b][RQ_T];
      const int rb = s_req[b][RQ_RB];
      const int chunks = rb > 0 ? (N + chunk_sel - 1) / chunk_sel : 0;
      s_req[b][RQ_CHUNKS] = chunks;
      s_req[b][RQ_ITEM0] = at;
      at += items_of(b, chunk_sel);
      most = max(most, chunks);
    }
    if (most) atomicMax(&s_max_chunks, most);
  }
  __syncthreads();
  if (tid == 0) {
    int items = all_items;
    s_chunk = chunk_sel;
    if (items > p.item_capacity) s_err |= MLA_VERIFY_DEVERR_CAPACITY;
    if (s_err & kMetaErrMask) items = 0;
    s_items = items;
  }
  __syncthreads();
  const int chunk = s_chunk;
  const int n_items = s_items;

  for (int b = tid; b < B; b += kMetaThreads) {
#pragma unroll
    for (int c = 0; c < 8; ++c) p.req[b * 8 + c] = s_req[b][c];
  }
  // work items: request, row block, key range [key0, key1) in combined order,
  // and for every split-partial workgroup its launch entry.  Workgroup g runs
  // on XCD g % 8 and takes item (g % 8) * per_xcd + g / 8, so the items of a
  // key range (consecutive, one per row block) share that XCD's L2; the entry
  // holds all the item's fields the workgroup needs, so it starts with one
  // load.
  const int per_xcd = (n_items + 7) >> 3;
  for (int g = tid; g < p.partial_grid; g += kMetaThreads) {
    const int it = (g & 7) * per_xcd + (g >> 3);
    int32_t* ln = p.launch + (size_t)g * 8;
    if ((g >> 3) >= per_xcd || it >= n_items) {
      *reinterpret_cast<i32x4*>(ln) = i32x4{-1, 0, 0, 0};
      continue;
    }
    int lo = 0, hi = B - 1;
    while (lo < hi) {  // last request whose first item is <= it
      const int mid = (lo + hi + 1) >> 1;
      if (s_req[mid][RQ_ITEM0] <= it) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int rbs = s_req[b][RQ_RB];
    const int local = it - s_req[b][RQ_ITEM0];
    const int c = local / rbs, rb = local % rbs;
    const int N = s_req[b][RQ_P] + s_req[b][RQ_T];
    const int key0 = c * chunk;
    const int key1 = min(N, key0 + chunk);
    const int rows = s_req[b][RQ_T] * H;
    const int row0 = rb * kRowsPerItem;
    const int nrows = min(kRowsPerItem, rows - row0);
    int32_t* e = p.items + (size_t)it * 8;
    *reinterpret_cast<i32x4*>(e) = i32x4{b, rb, c, key0};
    *reinterpret_cast<i32x4*>(e + 4) = i32x4{key1, row0, nrows, 0};
    *reinterpret_cast<i32x4*>(ln) = i32x4{it, key0, key1, row0};
    *reinterpret_cast<i32x4*>(ln + 4) =
        i32x4{nrows, s_req[b][RQ_P], s_req[b][RQ_Q0], s_req[b][RQ_KV0] + s_req[b][RQ_Q0]};
  }
  // per query token, for the merge: its request's first token, first item,
  // row blocks and key ranges (one 16-byte entry, so the merge reads no
  // request table)
  for (int t = tid; t < s_total_q; t += kMetaThreads) {
    int lo = 0, hi = B - 1;   // last request whose tokens start at or before t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_req[mid][RQ_Q0] <= t) lo = mid; else hi = mid - 1;
    }
    *reinterpret_cast<i32x4*>(p.tok + 4 * (size_t)t) =
        i32x4{s_req[lo][RQ_Q0], s_req[lo][RQ_ITEM0], s_req[lo][RQ_RB], s_req[lo][RQ_CHUNKS]};
  }
  if (tid == 0) {
    const int tq = s_total_q;
    p.hdr->err = s_err;
    p.hdr->n_items = n_items;
    p.hdr->total_q = tq;
    p.hdr->chunk_keys = chunk;
    p.hdr->batch = B;
    p.hdr->max_chunks = s_max_chunks;
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
// row: wave-uniform global address; lane_off: this lane's byte offset from it
__device__ __forceinline__ void dma16_row(const void* row, uint32_t lane_off, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(lane_off), "s"(row), "{m0}"(lds) : "memory");
}
// addr: this lane's global address
__device__ __forceinline__ void dma16(const void* addr, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(addr), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* addr, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(addr), "{m0}"(lds) : "memory");
}

// Row reductions over the four lane groups that hold one query row (lanes
// n, n+16, n+32, n+48): the gfx950 swaps exchange 16-lane rows (xor 16) and
// 32-lane halves (xor 32) in the VALU, with no LDS round trip.
__device__ __forceinline__ float group_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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
template <int kRowTilesMax>
__global__ __launch_bounds__(kPartialThreads, 1) void partial_kernel(KernelParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char s_v[kStages * kVSlotBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_r[kRopeSlots * kRopeSlotBytes];
  __shared__ bf16x8 s_p[2][kWaves][2][64];      // P(i) in buffer i & 1: row tile, hi/lo, lane
  __shared__ __attribute__((aligned(16))) int32_t s_idx[2][kIdxKeys];   // slot blocks (double buffered)
  __shared__ f32x4 s_alpha[2][16];              // [i & 1][n][rt]: rescale factor of row 16rt + n
  __shared__ uint32_t s_rescale[2];             // byte rt != 0 when row tile rt rescaled

  // Work items of one key range sit on one XCD: workgroup b is dispatched to
  // XCD b % 8, so XCD x gets the contiguous items [x*per, (x+1)*per) and the
  // row blocks that share a key range share that XCD's L2.
  // this workgroup's launch entry (written by the metadata launch, which
  // places the items of a key range on one XCD): item, key range, rows, and
  // its request's prefix length, first token and slot list
  const int bid = blockIdx.x;
  const i32x4 la = *reinterpret_cast<const i32x4*>(p.launch + (size_t)bid * 8);
  const i32x4 lb = *reinterpret_cast<const i32x4*>(p.launch + (size_t)bid * 8 + 4);
  const int item = la[0];
  if (item < 0) return;
  const int key0 = la[1], key1 = la[2], row0 = la[3];
  const int nrows = lb[0], P = lb[1], q0 = lb[2], slot0 = lb[3];
  const int H = p.num_heads;
  const int ntiles = (key1 - key0 + kKeysPerTile - 1) / kKeysPerTile;
  const int nrt = (nrows + 15) >> 4;            // row tiles with at least one row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool score_wave = wave < kWaves;
  const int r = score_wave ? wave : wave - kWaves;   // row tile (score) or dim eighth (PV)
  const int n = lane & 15, g = lane >> 4;

  const int r_local = 16 * r + n;
  // this request's checked slots, prefix keys then tree nodes
  const int32_t* kslots = p.slots + slot0;

  // ---- slots: blocks of kIdxKeys keys staged in LDS (double buffered) ----
  // The score waves copy the int32 slots of block b straight into LDS, lane
  // = key, with the tile loads.  Keys past the range end re-read the range's
  // last slot.  A slot of -1 (outside the pool) or -2 (a prefix key that a
  // checked full-row mask hides) reads slot 0 instead and poisons the item:
  // its rows become NaN.
  bool out_of_pool = false, hidden = false;
  auto issue_idx = [&](int blk) {
    const int j = min(key0 + blk * kIdxKeys + 64 * wave + lane, key1 - 1);
    dma4(kslots + j, lds_addr(&s_idx[blk & 1][64 * wave]));
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
    int s;   // score waves: the slot of key 8w + lane / 8 (its rope row);
             // PV waves: the slot of key 4r + (lane & 3)
  };
  auto read_slots = [&](int t) {
    const int blk = t / kTilesPerIdx;
    const int32_t* idx = s_idx[blk & 1] - (key0 + blk * kIdxKeys);
    const int jt = key0 + t * kKeysPerTile;
    const int j = score_wave ? min(jt + 8 * wave + (lane >> 3), key1 - 1) : jt + 4 * r + (lane & 3);
    return TileSlots{idx[j]};
  };
  const unsigned char* pool = reinterpret_cast<const unsigned char*>(p.kv_pool);
  const uint32_t row_bytes = (uint32_t)p.kv_row_stride * 2;
  // the loads of a tile one at a time, so that the roles can spread them
  // over their MFMA steps
  auto issue_key = [&](int t, const TileSlots& ts, int i) {
    // one key per load: the slot is wave-uniform, so the row address is
    // formed on the scalar unit
    const int kk = 4 * r + i;
    const int32_t v = __builtin_amdgcn_readlane(ts.s, i);
    hidden |= v == kSlotMaskedPrefix;
    out_of_pool |= v < 0 && v != kSlotMaskedPrefix;
    const unsigned char* row = pool + (uint64_t)(uint32_t)max(v, 0) * row_bytes;
    dma16_row(row, (uint32_t)(lane ^ vswz(kk)) * 16, lds_addr(s_v + (t % kStages) * kVSlotBytes + kk * kVStride));
  };
  auto issue_rope = [&](int t, const TileSlots& ts) {
    const int kk = 8 * wave + (lane >> 3);
    const unsigned char* row = pool + (uint64_t)(uint32_t)max(ts.s, 0) * row_bytes;
    const int unit = (lane & 7) ^ rswz(kk);
    dma16(row + 2 * kDv + unit * 16, lds_addr(s_r + (t % kRopeSlots) * kRopeSlotBytes + (8 * wave) * 128));
  };
  auto issue = [&](int t, const TileSlots& ts) {
    if (score_wave) {
      issue_rope(t, ts);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) issue_key(t, ts, i);
    }
  };
  const int loads_per_tile = score_wave ? 1 : 4;

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
  // Index block b lands before tile 8b - 5 (issued after tile 8b - 6), and
  // is first read with the slots of tile 8b in iteration 8b - 3; its buffer
  // was last read in iteration 8b - 12.  The waits below count tile loads
  // only: index loads in flight behind a tile make them wait a little longer,
  // never less.
  TileSlots next_slots{};
  // The slots of tiles 0..2 come straight from the staged list (the same
  // values, clamped to the range's last key, that the LDS blocks hold), so
  // the first gathers wait for one load instead of the first slot block and a
  // barrier.  The first LDS slot read (tile 3, iteration 0) follows A(0),
  // by which every score wave's first index load has landed.  Loads the
  // compiler issued (queries, these slots) are older than the tile loads, so
  // the tile waits only ever wait longer for them.
  TileSlots pre[3] = {};
  auto load_pre = [&]() {
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      if (t >= ntiles) break;
      const int jt = key0 + t * kKeysPerTile;
      const int j = min(score_wave ? jt + 8 * wave + (lane >> 3) : jt + 4 * r + (lane & 3), key1 - 1);
      pre[t] = TileSlots{kslots[j]};
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
  // what iteration i issues after A(i): tile i + 2, index block i / 8 + 1
  // (score waves, every 8th iteration) and the slots of tile i + 3
  auto after_a = [&](int i) {
    if (i + 2 < ntiles) issue(i + 2, next_slots);
    if (score_wave && i % kTilesPerIdx == 0 && i + kTilesPerIdx < ntiles) issue_idx(i / kTilesPerIdx + 1);
    if (i + 3 < ntiles) next_slots = read_slots(i + 3);
  };

  if (score_wave) {
    // ---- score waves: query rows 16r + n; rows are (node, head), heads fastest
    const bool row_ok = r_local < nrows;
    const bool s_active = r < nrt;
    // the first slot block is on its way while the queries load
    if (ntiles > 0) issue_idx(0);
    load_pre();
    bf16x8 qf[kDqk / 32];
    uint64_t anc;
    {
      const int rr = row0 + r_local;
      const int tok = q0 + rr / H, head = rr % H;
      const uint16_t* qrow = p.q + (int64_t)tok * p.q_stride_tok + (int64_t)head * p.q_stride_head;
#pragma unroll
      for (int ks = 0; ks < kDqk / 32; ++ks) {
        u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(qrow + ks * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
      anc = row_ok ? p.anc[tok] : 0ull;
    }
    float m_run = -INFINITY, l_run = 0.f;       // softmax state of this lane's row
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
      if (lane == 0) reinterpret_cast<uint8_t*>(&s_rescale[bf])[r] = 0;
    }
    prologue();

    for (int i = 0; i <= ntiles; ++i) {
      barrier_a(i);
      if (!s_active || i >= ntiles) {
        after_a(i);
        continue;
      }
      const bool more = i + 2 < ntiles;
      const unsigned char* vslot = s_v + (i % kStages) * kVSlotBytes;
      const unsigned char* rslot = s_r + (i % kRopeSlots) * kRopeSlotBytes;
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
      // scores in base-2 units; mask the range tail and invisible tree keys
      const bool need_mask = jt + kKeysPerTile > min(P, key1);
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v = sacc[kt][q] * p.sm_scale_log2;
          if (need_mask) {
            const int j = jt + 16 * kt + 4 * g + q;
            bool vis = j < key1;
            if (j >= P) vis = vis && ((anc >> (j - P)) & 1ull);
            v = vis ? v : -INFINITY;
          }
          sacc[kt][q] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = group_max(mx);
      // lazy rescale: move a row's reference max only when the tile max
      // exceeds it by more than 2^kRescaleSlack (then p <= 2^8 stays safe)
      const bool need = mx > m_run + kRescaleSlack;
      const bool any_need = __builtin_amdgcn_ballot_w64(need) != 0;
      float alpha = 1.f;
      if (any_need) {
        const float m_new = need ? mx : m_run;
        alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float rs = 0.f;
      bf16x8 phi, plo;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float pv = __builtin_amdgcn_exp2f(sacc[kt][q] - m_use);
          rs += pv;
          const __bf16 h = (__bf16)pv;
          phi[kt * 4 + q] = h;
          plo[kt * 4 + q] = (__bf16)(pv - (float)h);
        }
      }
      l_run += group_sum(rs);
      s_p[i & 1][r][0][lane] = phi;
      s_p[i & 1][r][1][lane] = plo;
      if (any_need && g == 0) s_alpha[i & 1][n][r] = alpha;
      if (lane == 0) reinterpret_cast<uint8_t*>(&s_rescale[i & 1])[r] = any_need;
    }
    out_of_pool = __syncthreads_or(out_of_pool);
    hidden = __syncthreads_or(hidden);
    const bool poison = out_of_pool || hidden;
    if (tid == 0 && poison)
      atomicOr(&p.hdr->err, (out_of_pool ? (uint32_t)MLA_VERIFY_DEVERR_SLOT_RANGE : 0u) |
                                (hidden ? (uint32_t)MLA_VERIFY_DEVERR_MASK_PREFIX : 0u));
    if (row_ok && g == 0) {
      float* pm = p.part_ml + ((size_t)item * kRowsPerItem + r_local) * 2;
      pm[0] = m_run;
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
    int v_lo[kDtPerWave];
    {
      const int v_key = 4 * g + (n >> 2);
#pragma unroll
      for (int dt = 0; dt < kDtPerWave; ++dt)
        v_lo[dt] = v_key * kVStride + (n & 1) * 8 + ((((kDvPerWave / 8) * r + 2 * dt + ((n >> 1) & 1)) ^ vswz(v_key)) << 4);
    }
    load_pre();
    prologue();
    // The PV waves run two tiles behind the score waves: iteration i
    // multiplies tile i - 2 with operands that are all in registers by then
    // (P(i - 2) and its rescale factors, read in iteration i - 1; V^T(i - 2),
    // read in iteration i - 2), and meanwhile reads P(i - 1) and V^T(i).
    // vt[s][dt] is the A operand for dims 64r + 16dt, keys kappa(g, 0..7), of
    // the tile with parity s.
    bf16x8 vt[2][kDtPerWave];
    bf16x8 ph[kWaves], pl[kWaves];
    uint32_t resc = 0;
    f32x4 alpha4 = f32x4{1.f, 1.f, 1.f, 1.f};
    auto v_operand = [&](const unsigned char* vslot, int dt) -> bf16x8 {
      const unsigned char* vb = vslot + v_lo[dt];
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MLAV_LDS(i16x4, vb));
      const i16x4 vc = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MLAV_LDS(i16x4, vb + 16 * kVStride));
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
    // rescale factors were loaded in this iteration.  No iteration follows
    // only to drain the two-tile lag.
    auto final_pv = [&](auto parity) {
      constexpr int sv = decltype(parity)::value;
#pragma unroll
      for (int rt = 0; rt < kWaves; ++rt) {
        if (rt < kRowTilesMax) {
          if ((resc >> (8 * rt)) & 0xffu) {
            const float alpha = alpha4[rt];
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
      const unsigned char* vslot = s_v + (i % kStages) * kVSlotBytes;
      const bool v_next = i < ntiles;              // V^T(i) to read
      const bool p_next = i >= 1 && i <= ntiles;   // P(i - 1) to read
      if (i < 2) {
        if (v_next) {
#pragma unroll
          for (int dt = 0; dt < kDtPerWave; ++dt) vt[sv][dt] = v_operand(vslot, dt);
        }
        if (p_next) {
          resc = s_rescale[(i - 1) & 1];
          alpha4 = s_alpha[(i - 1) & 1][n];
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
      const f32x4 alpha_cur = alpha4;
      if (p_next) {
        resc = s_rescale[(i - 1) & 1];
        alpha4 = s_alpha[(i - 1) & 1][n];
      }
      // PV of tile i - 2, one row tile at a time (row tiles without rows
      // carry P = 0, so there are no branches but the rare rescale; row tiles
      // past kRowTilesMax are left out at compile time); each P operand, once
      // used, is replaced by P(i - 1), and in the last pass each V^T operand
      // by V^T(i)
#pragma unroll
      for (int rt = 0; rt < kWaves; ++rt) {
        if (rt < kRowTilesMax) {
          if ((resc_cur >> (8 * rt)) & 0xffu) {
            const float alpha = alpha_cur[rt];
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
    hidden = __syncthreads_or(hidden);
  }
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
// the w wave results are combined the same way through LDS.  A row waits
// for about three memory round trips (header, plan entry, partials).
// Workgroups past the last row exit at once.
// ---------------------------------------------------------------------------
constexpr int kMergeUnroll = 8;
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(KernelParams p) {
  constexpr int kMW = kMergeThreads / 64;
  __shared__ f32x4 s_acc[kMW][2][64];
  __shared__ float s_m[kMW], s_l[kMW];
  const WsHeader* hdr = p.hdr;
  const uint32_t err = hdr->err;
  const int total_q = hdr->total_q;
  const int most = hdr->max_chunks;
  const int H = p.num_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int wpr = 1;   // waves per row
  while (wpr < kMW && wpr * kMergeUnroll < most) wpr <<= 1;
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
  i32x4 tk = i32x4{0, 0, 0, 0};   // q0, item0, row blocks, chunks
  if (live) tk = *reinterpret_cast<const i32x4*>(p.tok + 4 * (size_t)t);
  const int r = (t - tk[0]) * H + h;
  const int rb = r / kRowsPerItem, lr = r % kRowsPerItem;
  const int item0 = tk[1], rbs = tk[2], chunks = live ? tk[3] : 0;
  auto item_of = [&](int c) { return (size_t)(item0 + c * rbs + rb) * kRowsPerItem + lr; };

  // fold weights 2^(m_c - M) into a running (M, L, acc); a range with no
  // visible key (m_c = -inf) adds nothing
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

int launch_meta(const KernelParams& p, const mla_verify_layout_t& lay, void* stream) {
  hipLaunchKernelGGL(meta_kernel, dim3(lay.meta_grid), dim3(kMetaThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int launch_partial(const KernelParams& p, const mla_verify_layout_t& lay, void* stream) {
  // the most rows an item of this plan holds bound its 16-row tiles
  const int64_t rows = (int64_t)p.max_tree_nodes * p.num_heads;
  const int tiles = rows >= kRowsPerItem ? kWaves : (int)((rows + 15) / 16);
  if (tiles <= 1)
    hipLaunchKernelGGL(partial_kernel<1>, dim3(lay.partial_grid), dim3(kPartialThreads), 0, (hipStream_t)stream, p);
  else if (tiles == 2)
    hipLaunchKernelGGL(partial_kernel<2>, dim3(lay.partial_grid), dim3(kPartialThreads), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(partial_kernel<kWaves>, dim3(lay.partial_grid), dim3(kPartialThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int launch_merge(const KernelParams& p, const mla_verify_layout_t& lay, void* stream) {
  if (lay.merge_grid <= 0) return 0;
  hipLaunchKernelGGL(merge_kernel, dim3(lay.merge_grid), dim3(kMergeThreads), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace mlav
