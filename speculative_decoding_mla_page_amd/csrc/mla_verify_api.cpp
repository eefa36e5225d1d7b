// Host side of the C-ABI: plan arithmetic, workspace layout, argument checks
// and the two launches of a call.  Owns no device memory and keeps no state.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>

#include "mla_verify_internal.h"

using namespace mlav;

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

const PlanImpl* as_impl(const mla_verify_plan_t* plan) {
  if (!plan) return nullptr;
  const PlanImpl* impl = reinterpret_cast<const PlanImpl*>(plan);
  if (impl->magic != kPlanMagic || impl->abi_version != MLA_VERIFY_ABI_VERSION) return nullptr;
  return impl;
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

mla_verify_status_t check_args(const PlanImpl& pl, const mla_verify_args_t* a, const void* ws,
                               size_t ws_bytes) {
  if (!a) return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  const mla_verify_config_t& c = pl.cfg;
  if (a->batch_size < 0 || a->batch_size > c.max_batch) return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (!isfinite(a->sm_scale) || !(a->sm_scale > 0.f)) return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (!a->q || !a->kv_pool || !a->qo_indptr || !a->kv_indptr || !a->kv_indices ||
      !a->out_cache_loc || !a->custom_mask || !a->mask_indptr || !a->out)
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  // 16-byte vector loads of q / pool rows and 16-byte stores of out
  if (!aligned(a->q, 16) || a->q_stride_tok <= 0 || a->q_stride_head <= 0 ||
      a->q_stride_tok % 8 || a->q_stride_head % 8)
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (!aligned(a->kv_pool, 16) || a->kv_row_stride < kDqk || a->kv_row_stride % 8 ||
      a->num_slots <= 0)
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  // slots are carried as int32 and row offsets formed as 32-bit x 32-bit products
  if (a->num_slots > INT32_MAX || a->kv_row_stride > (INT32_MAX >> 1)) return MLA_VERIFY_ERR_UNSUPPORTED;
  if (!aligned(a->out, 16) || a->out_stride_tok <= 0 || a->out_stride_head <= 0 ||
      a->out_stride_tok % 4 || a->out_stride_head % 4)
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (a->lse && (!aligned(a->lse, 4) || a->lse_stride_tok <= 0))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  // 16-byte row copies of the draft rows into the pool
  if (a->kv_new && (!aligned(a->kv_new, 16) || a->kv_new_stride_tok < kDqk || a->kv_new_stride_tok % 8 ||
                    a->kv_new_stride_tok > (INT32_MAX >> 1)))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;

  if (!aligned(a->qo_indptr, 4) || !aligned(a->kv_indptr, 4) || !aligned(a->mask_indptr, 4))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (!aligned(a->kv_indices, c.kv_indices_dtype == MLA_VERIFY_I64 ? 8 : 4) ||
      !aligned(a->out_cache_loc, c.out_cache_loc_dtype == MLA_VERIFY_I64 ? 8 : 4))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (!ws || !aligned(ws, kAlign)) return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (ws_bytes < pl.layout.total_bytes) return MLA_VERIFY_ERR_WORKSPACE_TOO_SMALL;
  return MLA_VERIFY_OK;
}

KernelParams make_params(const PlanImpl& pl, const mla_verify_args_t* a, void* ws) {
  KernelParams p;
  memset(&p, 0, sizeof(p));
  const mla_verify_config_t& c = pl.cfg;
  const mla_verify_layout_t& l = pl.layout;
  unsigned char* base = static_cast<unsigned char*>(ws);
  p.batch = a->batch_size;
  p.num_heads = c.num_heads;
  p.sm_scale_log2 = a->sm_scale * 1.4426950408889634f;
  p.q = static_cast<const uint16_t*>(a->q);
  p.q_stride_tok = a->q_stride_tok;
  p.q_stride_head = a->q_stride_head;
  p.kv_pool = static_cast<const uint16_t*>(a->kv_pool);
  p.kv_row_stride = a->kv_row_stride;
  p.num_slots = a->num_slots;
  p.qo_indptr = a->qo_indptr;
  p.kv_indptr = a->kv_indptr;
  p.kv_indices = a->kv_indices;
  p.out_cache_loc = a->out_cache_loc;
  p.custom_mask = a->custom_mask;
  p.mask_indptr = a->mask_indptr;
  p.out = a->out;
  p.out_stride_tok = a->out_stride_tok;
  p.out_stride_head = a->out_stride_head;
  p.lse = a->lse;
  p.lse_stride_tok = a->lse_stride_tok;
  p.kv_new = reinterpret_cast<const uint16_t*>(a->kv_new);
  p.kv_new_stride_tok = a->kv_new_stride_tok;
  p.kv_idx64 = c.kv_indices_dtype == MLA_VERIFY_I64;
  p.ocl_idx64 = c.out_cache_loc_dtype == MLA_VERIFY_I64;
  p.max_q_tokens = c.max_q_tokens;
  p.max_tree_nodes = c.max_tree_nodes;
  p.max_kv_tokens = c.max_kv_tokens;
  p.target_items = l.target_items;
  p.item_capacity = l.item_capacity;
  p.flags = c.flags;
  p.hdr = reinterpret_cast<WsHeader*>(base + l.header_offset);
  p.req = reinterpret_cast<int32_t*>(base + l.request_offset);
  p.anc = reinterpret_cast<uint64_t*>(base + l.anc_offset);
  p.items = reinterpret_cast<int32_t*>(base + l.items_offset);
  p.part_o = reinterpret_cast<float*>(base + l.partial_o_offset);
  p.part_ml = reinterpret_cast<float*>(base + l.partial_ml_offset);
  p.stats = reinterpret_cast<mla_verify_compare_stats_t*>(base + l.stats_offset);
  p.tok = reinterpret_cast<int32_t*>(base + l.tokens_offset);
  p.errs = reinterpret_cast<int32_t*>(base + l.errors_offset);
  p.partial_grid = l.partial_grid;
  p.trace = (c.flags & MLA_VERIFY_FLAG_TRACE_KEYS) ? reinterpret_cast<int64_t*>(base + l.trace_offset)
                                                   : nullptr;
  return p;
}

}  // namespace

mla_verify_status_t mlav::check_call(const mla_verify_plan_t* plan, const mla_verify_args_t* args, const void* ws,
                                     size_t ws_bytes) {
  const PlanImpl* pl = as_impl(plan);
  if (!pl) return MLA_VERIFY_ERR_BAD_PLAN;
  return check_args(*pl, args, ws, ws_bytes);
}

extern "C" {

int32_t mla_verify_abi_version(void) { return MLA_VERIFY_ABI_VERSION; }

const char* mla_verify_status_string(mla_verify_status_t s) {
  switch (s) {
    case MLA_VERIFY_OK: return "ok";
    case MLA_VERIFY_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_VERIFY_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_VERIFY_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_VERIFY_ERR_LAUNCH: return "kernel launch failed";
    case MLA_VERIFY_ERR_BAD_PLAN: return "not a plan made by mla_verify_plan";
  }
  return "unknown status";
}

mla_verify_status_t mla_verify_plan(const mla_verify_config_t* cfg, mla_verify_plan_t* plan) {
  if (!cfg || !plan) return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  const mla_verify_config_t c = *cfg;
  if (c.num_heads < 1 || c.max_batch < 1 || c.max_q_tokens < 1 || c.max_tree_nodes < 1 ||
      c.max_kv_tokens < 0 || c.target_items < 0 || c.cu_count < 0)
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if ((c.kv_indices_dtype != MLA_VERIFY_I32 && c.kv_indices_dtype != MLA_VERIFY_I64) ||
      (c.out_cache_loc_dtype != MLA_VERIFY_I32 && c.out_cache_loc_dtype != MLA_VERIFY_I64))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (c.flags & ~(uint32_t)(MLA_VERIFY_FLAG_TRACE_KEYS | MLA_VERIFY_FLAG_MASK_FULL_ROWS |
                            MLA_VERIFY_FLAG_CHECK_PREFIX_MASK | MLA_VERIFY_FLAG_CONTIGUOUS_PREFIX))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  // the prefix check reads the prefix columns of full mask rows
  if ((c.flags & MLA_VERIFY_FLAG_CHECK_PREFIX_MASK) && !(c.flags & MLA_VERIFY_FLAG_MASK_FULL_ROWS))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 7; ++i)
    if (c.reserved[i]) return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (c.max_tree_nodes > MLA_VERIFY_MAX_TREE_NODES || c.max_batch > kMaxBatch)
    return MLA_VERIFY_ERR_UNSUPPORTED;
  // int32 key and row indices inside the kernels
  if (c.max_kv_tokens > (int64_t)INT32_MAX - c.max_q_tokens) return MLA_VERIFY_ERR_UNSUPPORTED;
  const int64_t max_rows = (int64_t)c.max_q_tokens * c.num_heads;
  if (max_rows > INT32_MAX / 2) return MLA_VERIFY_ERR_UNSUPPORTED;

  int32_t cu = c.cu_count;
  if (cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
      return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  }
  const int32_t target = c.target_items > 0 ? c.target_items : cu;

  PlanImpl impl;
  memset(&impl, 0, sizeof(impl));
  impl.magic = kPlanMagic;
  impl.abi_version = MLA_VERIFY_ABI_VERSION;
  impl.cfg = c;
  impl.cfg.cu_count = cu;
  mla_verify_layout_t& l = impl.layout;
  // every request adds at most one partly filled key range per row block
  const int64_t row_blocks_bound = (max_rows + kRowsPerItem - 1) / kRowsPerItem + c.max_batch;
  // room for two rounds of target items (the device-side plan may choose
  // shorter key ranges over two rounds when many short requests would leave
  // one round badly balanced), plus the partly filled ranges
  const int64_t capacity = 2 * (int64_t)target + row_blocks_bound;
  if (capacity > INT32_MAX / 2) return MLA_VERIFY_ERR_UNSUPPORTED;
  l.item_capacity = (int32_t)capacity;
  l.rows_per_item = kRowsPerItem;
  l.keys_per_tile = kKeysPerTile;
  l.target_items = target;
  // the split-partial launch: about one workgroup per target item (one per
  // compute unit), whole groups of 8 (one per XCD), enough that none runs
  // more than kMaxItemsPerWg items
  const int64_t per_xcd_max = (capacity + 7) / 8;
  const int64_t g8 = std::max<int64_t>((target + 7) / 8, (per_xcd_max + kMaxItemsPerWg - 1) / kMaxItemsPerWg);
  l.partial_grid = (int32_t)(8 * g8);
  l.merge_grid = (int32_t)max_rows;

  uint64_t off = 0;
  l.header_offset = off;
  off = align_up(off + sizeof(WsHeader));
  l.request_offset = off;
  off = align_up(off + (uint64_t)c.max_batch * 8 * sizeof(int32_t));
  l.anc_offset = off;
  off = align_up(off + (uint64_t)c.max_q_tokens * sizeof(uint64_t));
  l.items_offset = off;
  off = align_up(off + (uint64_t)capacity * 8 * sizeof(int32_t));
  l.partial_o_offset = off;
  off = align_up(off + (uint64_t)capacity * kRowsPerItem * kDv * sizeof(float));
  l.partial_ml_offset = off;
  off = align_up(off + (uint64_t)capacity * kRowsPerItem * 2 * sizeof(float));
  l.trace_offset = 0;
  if (c.flags & MLA_VERIFY_FLAG_TRACE_KEYS) {
    l.trace_offset = off;
    off = align_up(off + ((uint64_t)c.max_kv_tokens + c.max_q_tokens) * sizeof(int64_t));
  }
  l.stats_offset = off;
  off = align_up(off + sizeof(mla_verify_compare_stats_t));
  l.tokens_offset = off;
  off = align_up(off + (uint64_t)c.max_q_tokens * 4 * sizeof(int32_t));
  l.errors_offset = off;
  off = align_up(off + (uint64_t)l.partial_grid * sizeof(int32_t));
  l.total_bytes = off;

  memset(plan, 0, sizeof(*plan));
  memcpy(plan, &impl, sizeof(impl));
  return MLA_VERIFY_OK;
}

mla_verify_status_t mla_verify_workspace_size(const mla_verify_plan_t* plan, size_t* bytes) {
  const PlanImpl* pl = as_impl(plan);
  if (!pl) return MLA_VERIFY_ERR_BAD_PLAN;
  if (!bytes) return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  *bytes = (size_t)pl->layout.total_bytes;
  return MLA_VERIFY_OK;
}

mla_verify_status_t mla_verify_workspace_layout(const mla_verify_plan_t* plan,
                                                mla_verify_layout_t* layout) {
  const PlanImpl* pl = as_impl(plan);
  if (!pl) return MLA_VERIFY_ERR_BAD_PLAN;
  if (!layout) return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  *layout = pl->layout;
  return MLA_VERIFY_OK;
}

mla_verify_status_t mla_verify_run_phase(const mla_verify_plan_t* plan, const mla_verify_args_t* args,
                                         void* workspace, size_t workspace_bytes, void* stream,
                                         int32_t phase) {
  const PlanImpl* pl = as_impl(plan);
  if (!pl) return MLA_VERIFY_ERR_BAD_PLAN;
  if (phase < 0 || phase > 1) return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  const mla_verify_status_t st = check_args(*pl, args, workspace, workspace_bytes);
  if (st != MLA_VERIFY_OK) return st;
  const KernelParams p = make_params(*pl, args, workspace);
  const int rc = phase == 0 ? launch_partial(p, pl->layout, stream) : launch_merge(p, pl->layout, stream);
  return rc == 0 ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}

mla_verify_status_t mla_verify_compare(const mla_verify_plan_t* plan, const mla_verify_args_t* args,
                                       const float* ref_out, int64_t ref_out_stride_tok,
                                       int64_t ref_out_stride_head, const float* ref_lse,
                                       int64_t ref_lse_stride_tok, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const PlanImpl* pl = as_impl(plan);
  if (!pl) return MLA_VERIFY_ERR_BAD_PLAN;
  const mla_verify_status_t st = check_args(*pl, args, workspace, workspace_bytes);
  if (st != MLA_VERIFY_OK) return st;
  // the reference is read like out: 16-byte rows
  if (!ref_out || !aligned(ref_out, 16) || ref_out_stride_tok <= 0 || ref_out_stride_head <= 0 ||
      ref_out_stride_tok % 4 || ref_out_stride_head % 4)
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (ref_lse && (!args->lse || !aligned(ref_lse, 4) || ref_lse_stride_tok <= 0))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  KernelParams p = make_params(*pl, args, workspace);
  p.ref_out = ref_out;
  p.ref_out_stride_tok = ref_out_stride_tok;
  p.ref_out_stride_head = ref_out_stride_head;
  p.ref_lse = ref_lse;
  p.ref_lse_stride_tok = ref_lse_stride_tok;
  return launch_compare(p, pl->layout, stream) == 0 ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}

mla_verify_status_t mla_verify_compact(const mla_verify_plan_t* plan, const mla_verify_args_t* args,
                                       const int64_t* dst_start, int32_t* error_word, void* stream) {
  const PlanImpl* pl = as_impl(plan);
  if (!pl) return MLA_VERIFY_ERR_BAD_PLAN;
  if (!args || !dst_start || !error_word || !aligned(dst_start, 8) || !aligned(error_word, 4))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  const mla_verify_config_t& c = pl->cfg;
  if (args->batch_size < 0 || args->batch_size > c.max_batch || !args->kv_pool || !args->kv_indptr ||
      !args->kv_indices || !aligned(args->kv_pool, 16) || args->kv_row_stride < kDqk ||
      args->kv_row_stride % 8 || args->num_slots <= 0 || !aligned(args->kv_indptr, 4) ||
      !aligned(args->kv_indices, c.kv_indices_dtype == MLA_VERIFY_I64 ? 8 : 4))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  if (args->num_slots > INT32_MAX || args->kv_row_stride > (INT32_MAX >> 1)) return MLA_VERIFY_ERR_UNSUPPORTED;
  KernelParams p;
  memset(&p, 0, sizeof(p));
  p.batch = args->batch_size;
  p.kv_pool = reinterpret_cast<const uint16_t*>(args->kv_pool);
  p.kv_row_stride = args->kv_row_stride;
  p.num_slots = args->num_slots;
  p.kv_indptr = args->kv_indptr;
  p.kv_indices = args->kv_indices;
  p.kv_idx64 = c.kv_indices_dtype == MLA_VERIFY_I64;
  p.max_kv_tokens = c.max_kv_tokens;
  return launch_compact(p, dst_start, error_word, stream) == 0 ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}

mla_verify_status_t mla_verify_run(const mla_verify_plan_t* plan, const mla_verify_args_t* args,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  const PlanImpl* pl = as_impl(plan);
  if (!pl) return MLA_VERIFY_ERR_BAD_PLAN;
  const mla_verify_status_t st = check_args(*pl, args, workspace, workspace_bytes);
  if (st != MLA_VERIFY_OK) return st;
  const KernelParams p = make_params(*pl, args, workspace);
  if (launch_partial(p, pl->layout, stream) != 0) return MLA_VERIFY_ERR_LAUNCH;
  if (launch_merge(p, pl->layout, stream) != 0) return MLA_VERIFY_ERR_LAUNCH;
  return MLA_VERIFY_OK;
}

}  // extern "C"
