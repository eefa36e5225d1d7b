// Internal definitions shared by the host planner and the gfx950 kernels.
#pragma once

#include <stdint.h>

#include "mla_verify.h"

namespace mlav {

constexpr int kDqk = MLA_VERIFY_D_QK;      // 576
constexpr int kDv = MLA_VERIFY_D_V;        // 512
constexpr int kKeysPerTile = 32;           // keys staged in LDS per inner step
constexpr int kWaves = 4;                  // waves per workgroup (one per SIMD)
constexpr int kRowTiles = 1;               // 16-row MFMA tiles of query rows per wave
constexpr int kRowsPerWave = 16 * kRowTiles;
constexpr int kRowsPerItem = kWaves * kRowsPerWave;  // query rows per work item
constexpr int kStages = 3;                 // LDS slots of key tiles (V part)
constexpr int kIdxKeys = 256;              // slots staged per index block (8 tiles)
constexpr int kPVWaves = 8;                // PV waves per workgroup (64 output dims each)
constexpr int kPartialThreads = (kWaves + kPVWaves) * 64;   // score waves + PV waves
constexpr int kMergeThreads = 512;         // 8 waves per output row, each lane 8 of the 512 dims
constexpr int kMinChunkKeys = 128;         // shortest key range of a work item
constexpr int kMaxItemsPerWg = 4;          // work items one split-partial workgroup runs, at most
constexpr int kMaxBatch = 1024;            // per-request plan tables live in LDS of every split-partial workgroup
constexpr uint32_t kPlanMagic = 0x5641'4c4du;  // "MLAV"

// request table columns (int32 x 8 per request)
enum { RQ_P = 0, RQ_T, RQ_Q0, RQ_KV0, RQ_RB, RQ_CHUNKS, RQ_ITEM0, RQ_MASK0 };
// work-item table columns (int32 x 8 per item)
enum { IT_B = 0, IT_RB, IT_CHUNK, IT_KEY0, IT_KEY1, IT_ROW0, IT_NROWS };

struct WsHeader {
  uint32_t err;         // every device error bit of the call (written by the merge launch)
  int32_t n_items;
  int32_t total_q;
  int32_t chunk_keys;
  int32_t batch;
  int32_t max_chunks;   // key ranges of the request with the most
  uint32_t err_meta;    // the metadata checks' bits alone (written by the split-partial launch)
  int32_t pad;
};

constexpr uint32_t kMetaErrMask = MLA_VERIFY_DEVERR_QO_INDPTR | MLA_VERIFY_DEVERR_KV_INDPTR |
                                  MLA_VERIFY_DEVERR_TREE_SIZE | MLA_VERIFY_DEVERR_MASK_INDPTR |
                                  MLA_VERIFY_DEVERR_CAPACITY;
// a key's slot as the split-partial kernel carries it: >= 0 a pool slot; a
// slot outside the pool is kSlotBad (the item is poisoned and reads slot 0)
constexpr int32_t kSlotBad = -1;

struct PlanImpl {
  uint32_t magic;
  int32_t abi_version;
  mla_verify_config_t cfg;
  mla_verify_layout_t layout;
};
static_assert(sizeof(PlanImpl) <= sizeof(mla_verify_plan_t), "plan does not fit the opaque value");

// Everything a kernel needs, passed by value.
struct KernelParams {
  // call arguments
  int32_t batch;
  int32_t num_heads;
  float sm_scale_log2;          // sm_scale * log2(e): scores kept in base-2 units
  const uint16_t* q;
  int64_t q_stride_tok;
  int64_t q_stride_head;
  const uint16_t* kv_pool;
  int64_t kv_row_stride;
  int64_t num_slots;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const void* kv_indices;
  const void* out_cache_loc;
  const uint8_t* custom_mask;
  const int32_t* mask_indptr;
  float* out;
  int64_t out_stride_tok;
  int64_t out_stride_head;
  float* lse;
  int64_t lse_stride_tok;
  const uint16_t* kv_new;       // optional draft rows, stored into the pool before they are gathered
  int64_t kv_new_stride_tok;
  // plan
  int32_t kv_idx64;
  int32_t ocl_idx64;
  int32_t max_q_tokens;
  int32_t max_tree_nodes;
  int64_t max_kv_tokens;
  int32_t target_items;
  int32_t item_capacity;
  uint32_t flags;
  // workspace regions
  WsHeader* hdr;
  int32_t* req;
  uint64_t* anc;
  int32_t* tok;   // [max_q_tokens][4]: request's first token, first item, row blocks, key ranges
  int32_t* errs;  // [partial_grid]: device error bits found by each split-partial workgroup
  int32_t partial_grid;
  int32_t* items;
  float* part_o;
  float* part_ml;
  int64_t* trace;
  mla_verify_compare_stats_t* stats;
  // shadow comparison only
  const float* ref_out;
  int64_t ref_out_stride_tok;
  int64_t ref_out_stride_head;
  const float* ref_lse;
  int64_t ref_lse_stride_tok;
};

// run()'s host-side checks of a plan and its call arguments (no HIP call)
mla_verify_status_t check_call(const mla_verify_plan_t* plan, const mla_verify_args_t* args, const void* ws,
                               size_t ws_bytes);

int launch_partial(const KernelParams& p, const mla_verify_layout_t& lay, void* stream);
int launch_merge(const KernelParams& p, const mla_verify_layout_t& lay, void* stream);
int launch_compare(const KernelParams& p, const mla_verify_layout_t& lay, void* stream);
int launch_compact(const KernelParams& p, const int64_t* dst_start, int32_t* error_word, void* stream);

}  // namespace mlav
