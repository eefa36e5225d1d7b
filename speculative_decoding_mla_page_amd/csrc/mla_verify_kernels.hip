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

#include "mla_verify_internal.h"

namespace mlav {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// LDS layout of one staged key tile (kKeysPerTile keys):
//   s_k : key-major copy, row = key, 576 bf16 + 16 bytes of padding, read as the
//         A operand of S^T = K.Q^T (16 contiguous bytes of one key per lane).
//   s_vt: dim-major copy of V = dims [0,512): row = dim, 4 key groups x 8 keys
//         + 16 bytes of padding, read as the A operand of O^T = V^T.P^T.
constexpr int kKStride = kDqk * 2 + 16;                  // 1168 bytes
constexpr int kVtStride = kKeysPerTile * 2 + 16;         // 80 bytes
constexpr int kSkBytes = kKeysPerTile * kKStride;        // 37376
constexpr int kSvtBytes = kDv * kVtStride;               // 40960

// Key order inside a 32-key tile for the PV product.  Lane group g (lanes
// 16g..16g+15) feeds keys kappa(g, 0..7) = {4g..4g+3, 16+4g..16+4g+3} as its
// eight K-dimension slots; these are exactly the keys whose scores the same
// lanes hold in the S^T accumulators (rows 4g+i of each 16-key output tile),
// so P moves from the softmax to the PV operand without any data exchange.
__device__ __forceinline__ int kappa(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

__device__ __forceinline__ int64_t load_index(const void* base, int64_t i, int is64) {
  return is64 ? reinterpret_cast<const int64_t*>(base)[i]
              : static_cast<int64_t>(reinterpret_cast<const int32_t*>(base)[i]);
}

// Slot of key j (combined order: prefix then tree) of a request, or -1 past the range.
__device__ __forceinline__ int64_t key_slot(const KernelParams& p, int j, int key1, int P, int kv0,
                                            int q0) {
  if (j >= key1) return -1;
  if (j < P) return load_index(p.kv_indices, (int64_t)kv0 + j, p.kv_idx64);
  return load_index(p.out_cache_loc, (int64_t)q0 + (j - P), p.ocl_idx64);
}

// ---------------------------------------------------------------------------
// metadata build: one workgroup
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMetaThreads) void meta_kernel(KernelParams p) {
  __shared__ int32_t s_req[kMaxBatch][8];
  __shared__ uint32_t s_err;
  __shared__ long long s_work;
  __shared__ int32_t s_chunk;
  __shared__ int32_t s_items;
  const int tid = threadIdx.x;
  const int B = p.batch;
  const int H = p.num_heads;
  if (tid == 0) {
    s_err = 0;
    s_work = 0;
  }
  __syncthreads();

  // per-request lengths and checks (prefix length = kv_indptr[b+1] - kv_indptr[b])
  uint32_t err = 0;
  long long work = 0;
  for (int b = tid; b < B; b += kMetaThreads) {
    const int q0 = p.qo_indptr[b], q1 = p.qo_indptr[b + 1];
    const int k0 = p.kv_indptr[b], k1 = p.kv_indptr[b + 1];
    const int m0 = p.mask_indptr[b], m1 = p.mask_indptr[b + 1];
    const int T = q1 - q0, P = k1 - k0;
    if (q0 < 0 || T < 0 || q1 > p.max_q_tokens || (b == 0 && q0 != 0)) err |= MLA_VERIFY_DEVERR_QO_INDPTR;
    if (k0 < 0 || P < 0 || (long long)k1 > p.max_kv_tokens) err |= MLA_VERIFY_DEVERR_KV_INDPTR;
    if (T > p.max_tree_nodes) err |= MLA_VERIFY_DEVERR_TREE_SIZE;
    if (m0 < 0 || (long long)(m1 - m0) != (long long)T * T) err |= MLA_VERIFY_DEVERR_MASK_INDPTR;
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
  }
  if (err) atomicOr(&s_err, err);
  if (work) atomicAdd(reinterpret_cast<unsigned long long*>(&s_work), (unsigned long long)work);
  __syncthreads();

  // key-range length shared by all requests: total (row block x key) work cut
  // into about target_items pieces, rounded up to whole tiles
  if (tid == 0) {
    const long long per = (s_work + p.target_items - 1) / p.target_items;
    long long chunk = ((per + kKeysPerTile - 1) / kKeysPerTile) * kKeysPerTile;
    if (chunk < kKeysPerTile) chunk = kKeysPerTile;
    if (chunk > (1LL << 30)) chunk = 1LL << 30;
    s_chunk = (int)chunk;
    int items = 0;
    for (int b = 0; b < B; ++b) {
      const int N = s_req[b][RQ_P] + s_req[b][RQ_T];
      const int rb = s_req[b][RQ_RB];
      const int chunks = rb > 0 ? (N + (int)chunk - 1) / (int)chunk : 0;
      s_req[b][RQ_CHUNKS] = chunks;
      s_req[b][RQ_ITEM0] = items;
      items += rb * chunks;
    }
    if (items > p.item_capacity) s_err |= MLA_VERIFY_DEVERR_CAPACITY;
    if (s_err & kMetaErrMask) items = 0;
    s_items = items;
  }
  __syncthreads();
  const bool bad = (s_err & kMetaErrMask) != 0;
  const int chunk = s_chunk;
  const int n_items = s_items;

  for (int b = tid; b < B; b += kMetaThreads) {
#pragma unroll
    for (int c = 0; c < 8; ++c) p.req[b * 8 + c] = s_req[b][c];
  }
  // work items: request, row block, key range [key0, key1) in combined order
  for (int it = tid; it < n_items; it += kMetaThreads) {
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
    int32_t* e = p.items + (size_t)it * 8;
    e[IT_B] = b;
    e[IT_RB] = rb;
    e[IT_CHUNK] = c;
    e[IT_KEY0] = key0;
    e[IT_KEY1] = key1;
    e[IT_ROW0] = rb * kRowsPerItem;
    e[IT_NROWS] = min(kRowsPerItem, rows - rb * kRowsPerItem);
    e[7] = 0;
  }
  // packed tree visibility: bit k of node i's word = mask[i][k] != 0
  const int total_q = bad ? 0 : (B > 0 ? p.qo_indptr[B] : 0);
  for (int t = tid; t < total_q; t += kMetaThreads) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_req[mid][RQ_Q0] <= t) lo = mid; else hi = mid - 1;
    }
    // with monotone indptrs the last request starting at or before t holds t
    const int b = lo;
    const int T = s_req[b][RQ_T];
    const int i = t - s_req[b][RQ_Q0];
    const uint8_t* row = p.custom_mask + s_req[b][RQ_MASK0] + (size_t)i * T;
    uint64_t w = 0;
    for (int k = 0; k < T; ++k) w |= (uint64_t)(row[k] != 0) << k;
    p.anc[t] = w;
  }
  if (tid == 0) {
    int tq = B > 0 ? p.qo_indptr[B] : 0;
    tq = tq < 0 ? 0 : (tq > p.max_q_tokens ? p.max_q_tokens : tq);
    p.hdr->err = s_err;
    p.hdr->n_items = n_items;
    p.hdr->total_q = tq;
    p.hdr->chunk_keys = chunk;
    p.hdr->batch = B;
  }
}

// ---------------------------------------------------------------------------
// split partial: one workgroup (4 waves x 16 query rows) per work item
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);  // lo16(x) | lo16(y) << 16
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);  // hi16(x) | hi16(y) << 16
}

__global__ __launch_bounds__(kPartialThreads, 1) void partial_kernel(KernelParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char s_k[kSkBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_vt[kSvtBytes];

  const int item = blockIdx.x;
  if (item >= p.hdr->n_items) return;
  const int32_t* e = p.items + (size_t)item * 8;
  const int b = e[IT_B], rb = e[IT_RB], key0 = e[IT_KEY0], key1 = e[IT_KEY1];
  const int nrows = e[IT_NROWS], row0 = e[IT_ROW0];
  const int32_t* rq = p.req + b * 8;
  const int P = rq[RQ_P], q0 = rq[RQ_Q0], kv0 = rq[RQ_KV0];
  const int H = p.num_heads;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;

  // this lane's query row: rows are (node, head) pairs, heads fastest
  const int r_local = wave * kRowsPerWave + n;
  const bool row_ok = r_local < nrows;
  const int r = row0 + r_local;
  const int tok = q0 + r / H, head = r % H;
  bf16x8 qf[kDqk / 32];
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const uint16_t* qrow = p.q + (int64_t)tok * p.q_stride_tok + (int64_t)head * p.q_stride_head;
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) {
      u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(qrow + ks * 32 + g * 8) : zero;
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const uint64_t anc = row_ok ? p.anc[tok] : 0ull;
  const bool wave_active = wave * kRowsPerWave < nrows;
  const bool trace = (p.flags & MLA_VERIFY_FLAG_TRACE_KEYS) && rb == 0;
  const int64_t trace0 = (int64_t)kv0 + q0;

  f32x4 o[kDv / 16];
#pragma unroll
  for (int dt = 0; dt < kDv / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  bool poison = false;

  // gather assignment: wave w loads keys kappa(w, 0..7), lane = 16-byte column
  // of dims [0, 512); every thread also loads one 16-byte piece of the rope dims
  const int dg = lane;
  const int kr = tid >> 3, rg = tid & 7;
  u32x4 gm[8];
  u32x4 gr;

  auto gather = [&](int t0) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = t0 + kappa(wave, jj);
      const int64_t slot = key_slot(p, j, key1, P, kv0, q0);
      const bool ok = slot >= 0 && slot < p.num_slots;
      if (!ok && j < key1) poison = true;
      gm[jj] = ok ? *reinterpret_cast<const u32x4*>(p.kv_pool + slot * p.kv_row_stride + dg * 8)
                  : u32x4{0u, 0u, 0u, 0u};
    }
    const int j = t0 + kr;
    const int64_t slot = key_slot(p, j, key1, P, kv0, q0);
    const bool ok = slot >= 0 && slot < p.num_slots;
    if (!ok && j < key1) poison = true;
    gr = ok ? *reinterpret_cast<const u32x4*>(p.kv_pool + slot * p.kv_row_stride + kDv + rg * 8)
            : u32x4{0u, 0u, 0u, 0u};
    if (trace && rg == 0 && j < key1) p.trace[trace0 + j] = slot;
  };

  auto stage = [&]() {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      *reinterpret_cast<u32x4*>(s_k + kappa(wave, jj) * kKStride + dg * 16) = gm[jj];
    *reinterpret_cast<u32x4*>(s_k + kr * kKStride + kDv * 2 + rg * 16) = gr;
    // 8 keys x 8 dims -> 8 dims x 8 keys
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int w = d >> 1;
      u32x4 v;
      if ((d & 1) == 0) {
        v[0] = perm_lo(gm[0][w], gm[1][w]);
        v[1] = perm_lo(gm[2][w], gm[3][w]);
        v[2] = perm_lo(gm[4][w], gm[5][w]);
        v[3] = perm_lo(gm[6][w], gm[7][w]);
      } else {
        v[0] = perm_hi(gm[0][w], gm[1][w]);
        v[1] = perm_hi(gm[2][w], gm[3][w]);
        v[2] = perm_hi(gm[4][w], gm[5][w]);
        v[3] = perm_hi(gm[6][w], gm[7][w]);
      }
      *reinterpret_cast<u32x4*>(s_vt + (dg * 8 + d) * kVtStride + wave * 16) = v;
    }
  };

  gather(key0);
  for (int t0 = key0; t0 < key1; t0 += kKeysPerTile) {
    __syncthreads();  // previous tile's LDS reads are done
    stage();
    __syncthreads();
    if (t0 + kKeysPerTile < key1) gather(t0 + kKeysPerTile);

    if (wave_active) {
      // S^T tile: 32 keys x 16 rows, two 16-key MFMA tiles, K-dim 576
      f32x4 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const unsigned char* kp = s_k + (16 * kt + n) * kKStride + g * 16;
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kp + ks * 64);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], acc, 0, 0, 0);
        }
        s[kt] = acc;
      }
      // scale to base-2 units, mask the range tail and invisible tree keys
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = t0 + 16 * kt + 4 * g + i;
          float v = s[kt][i] * p.sm_scale_log2;
          bool vis = j < key1;
          if (j >= P) vis = vis && ((anc >> (j - P)) & 1ull);
          v = vis ? v : -INFINITY;
          s[kt][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float rs = 0.f;
      bf16x8 phi, plo;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = exp2f(s[kt][i] - m_use);
          rs += pv;
          const __bf16 h = (__bf16)pv;
          const __bf16 lo = (__bf16)(pv - (float)h);
          phi[kt * 4 + i] = h;
          plo[kt * 4 + i] = lo;
        }
      }
      rs += __shfl_xor(rs, 16);
      rs += __shfl_xor(rs, 32);
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < kDv / 16; ++dt) o[dt] *= alpha;
      // O^T += V^T . P^T with P split into bf16 hi + lo
#pragma unroll
      for (int dt = 0; dt < kDv / 16; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(s_vt + (16 * dt + n) * kVtStride + g * 16);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, o[dt], 0, 0, 0);
      }
    }
  }

  poison = __syncthreads_or(poison);
  if (poison && tid == 0) atomicOr(&p.hdr->err, (uint32_t)MLA_VERIFY_DEVERR_SLOT_RANGE);
  if (row_ok) {
    float* po = p.part_o + ((size_t)item * kRowsPerItem + r_local) * kDv;
#pragma unroll
    for (int dt = 0; dt < kDv / 16; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g) = o[dt];
    if (g == 0) {
      float* pm = p.part_ml + ((size_t)item * kRowsPerItem + r_local) * 2;
      pm[0] = m_run;
      pm[1] = poison ? NAN : l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// merge: one workgroup of 128 lanes per query row (token, head)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(KernelParams p) {
  __shared__ float s_red[kMergeThreads / 64];
  const int H = p.num_heads;
  const int row = blockIdx.x;
  const int t = row / H, h = row % H;
  const WsHeader* hdr = p.hdr;
  if (t >= hdr->total_q) return;
  const int tid = threadIdx.x;
  float* outp = p.out + (int64_t)t * p.out_stride_tok + (int64_t)h * p.out_stride_head;
  float* lsep = p.lse ? p.lse + (int64_t)t * p.lse_stride_tok + h : nullptr;
  if (hdr->err & kMetaErrMask) {
    *reinterpret_cast<f32x4*>(outp + 4 * tid) = f32x4{NAN, NAN, NAN, NAN};
    if (lsep && tid == 0) *lsep = NAN;
    return;
  }
  // request of token t
  const int B = hdr->batch;
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.req[mid * 8 + RQ_Q0] <= t) lo = mid; else hi = mid - 1;
  }
  const int b = lo;  // last request starting at or before t: it holds t
  const int32_t* rq = p.req + b * 8;
  const int r = (t - rq[RQ_Q0]) * H + h;
  const int rb = r / kRowsPerItem, lr = r % kRowsPerItem;
  const int chunks = rq[RQ_CHUNKS], rbs = rq[RQ_RB], base = rq[RQ_ITEM0];

  float mloc = -INFINITY;
  for (int c = tid; c < chunks; c += kMergeThreads) {
    const int it = base + c * rbs + rb;
    mloc = fmaxf(mloc, p.part_ml[((size_t)it * kRowsPerItem + lr) * 2]);
  }
  for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = mloc;
  __syncthreads();
  float mstar = s_red[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) mstar = fmaxf(mstar, s_red[w]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (mstar != -INFINITY) {
    for (int c = 0; c < chunks; ++c) {
      const int it = base + c * rbs + rb;
      const float* pm = p.part_ml + ((size_t)it * kRowsPerItem + lr) * 2;
      const float w = exp2f(pm[0] - mstar);
      L += w * pm[1];
      const f32x4 v = *reinterpret_cast<const f32x4*>(p.part_o + ((size_t)it * kRowsPerItem + lr) * kDv + 4 * tid);
      acc += w * v;
    }
  }
  f32x4 res;
  float lse;
  if (mstar == -INFINITY) {
    res = f32x4{0.f, 0.f, 0.f, 0.f};
    lse = -INFINITY;
  } else {
    const float inv = 1.f / L;
    res = acc * inv;
    lse = (mstar + log2f(L)) * 0.69314718055994531f;
  }
  *reinterpret_cast<f32x4*>(outp + 4 * tid) = res;
  if (lsep && tid == 0) *lsep = lse;
}

// ---------------------------------------------------------------------------
int launch_meta(const KernelParams& p, const mla_verify_layout_t& lay, void* stream) {
  (void)lay;
  hipLaunchKernelGGL(meta_kernel, dim3(1), dim3(kMetaThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int launch_partial(const KernelParams& p, const mla_verify_layout_t& lay, void* stream) {
  hipLaunchKernelGGL(partial_kernel, dim3(lay.partial_grid), dim3(kPartialThreads), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int launch_merge(const KernelParams& p, const mla_verify_layout_t& lay, void* stream) {
  if (lay.merge_grid <= 0) return 0;
  hipLaunchKernelGGL(merge_kernel, dim3(lay.merge_grid), dim3(kMergeThreads), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace mlav
