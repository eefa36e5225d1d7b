/*
 * mla_verify.h - tree-masked MLA verify attention over a page_size=1 latent KV
 * pool, for AMD Instinct MI355X (gfx950).
 *
 * One call computes, for every draft-tree query token of every request in a
 * segmented batch and for each of H heads, an exact softmax attention over
 *   (1) the request's prefix latent rows, read from a scattered pool through
 *       kv_indptr / kv_indices with one token per page ("The Integration Chasm",
 *       The Decision: Adapt the Kernel, Not the System), all visible, then
 *   (2) the request's own draft-tree rows, already written to the pool at
 *       out_cache_loc ("The Launch Wrapper", The KV Cache Ordering Insight),
 *       visible where the request's custom mask says so,
 * and reduces V = the first 512 of the 576 latent dims (the other 64 are the
 * rope part and only enter Q.K^T).
 *
 * Contract (from "The Capture-Safe Kernel", The Core Problem and Decisions 1-6):
 *   - the library consumes the serving framework's six metadata buffers as raw
 *     device pointers and derives prefix lengths, slots and mask offsets on the
 *     device (Decisions 1, 2, 5);
 *   - the launch grid depends on the plan only, never on buffer contents
 *     (Decision 3), so a captured graph stays valid while the buffers' contents
 *     change between replays (Decision 6);
 *   - all scratch lives in a caller-allocated workspace (Decision 4): run never
 *     allocates, synchronises, reads device memory on the host or creates
 *     temporaries, so it may be recorded into a hipGraph.
 *
 * Ownership: every pointer in mla_verify_args_t and the workspace is owned by
 * the caller and must stay valid until the work enqueued on `stream` ends.  The
 * library keeps no global mutable state; a plan is a plain value (copyable, no
 * destroy call).  Concurrent calls must use distinct workspaces.
 *
 * Errors: every entry point returns a status and checks host-visible arguments
 * only.  Problems found on the device (inconsistent indptrs, a tree larger than
 * the plan allows, a slot outside the pool) set bits of the error word at the
 * start of the workspace (mla_verify_layout_t.header_offset, complete once the
 * call has run) and the affected output rows are written as NaN; the caller
 * reads the word after its own sync.
 */
#ifndef MLA_VERIFY_H_
#define MLA_VERIFY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_VERIFY_ABI_VERSION 7
#define MLA_VERIFY_D_QK 576          /* latent width used by Q.K^T (512 + 64 rope) */
#define MLA_VERIFY_D_V 512           /* V = latent dims [0, 512) */
#define MLA_VERIFY_MAX_TREE_NODES 64 /* tree visibility is packed into one 64-bit word */
/* bytes of the device array mla_verify_run_static uses as its workspace (per GPU, held until the
   process ends) */
#define MLA_VERIFY_STATIC_SCRATCH_BYTES (96u << 20)

typedef enum {
  MLA_VERIFY_OK = 0,
  MLA_VERIFY_ERR_INVALID_ARGUMENT = 1, /* null / misaligned pointer, bad size or stride */
  MLA_VERIFY_ERR_UNSUPPORTED = 2,      /* a configuration the library does not implement */
  MLA_VERIFY_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_VERIFY_ERR_LAUNCH = 4,           /* the HIP runtime refused a launch */
  MLA_VERIFY_ERR_BAD_PLAN = 5          /* plan not produced by mla_verify_plan */
} mla_verify_status_t;

/* index dtypes */
enum { MLA_VERIFY_I32 = 0, MLA_VERIFY_I64 = 1 };

/* config flags */
enum {
  /* record every gathered slot in the workspace trace region (for bit-exact
     checks of the gather); costs one extra store per key */
  MLA_VERIFY_FLAG_TRACE_KEYS = 1u,
  /* custom_mask holds a full row per tree node: request b's block is
     T_b x (P_b + T_b), row-major, columns = its prefix keys then its tree
     nodes (the layout a serving framework's tree verify passes), and
     mask_indptr[b+1] - mask_indptr[b] = T_b * (P_b + T_b).  Only the tree
     columns are read: the prefix stays visible to every node. */
  MLA_VERIFY_FLAG_MASK_FULL_ROWS = 2u,
  /* with MLA_VERIFY_FLAG_MASK_FULL_ROWS: check that every prefix column is
     nonzero; a zero marks the keys it covers, the work items that gather them
     write NaN rows and set MLA_VERIFY_DEVERR_MASK_PREFIX.  Costs one mask byte
     read per (tree node, prefix key). */
  MLA_VERIFY_FLAG_CHECK_PREFIX_MASK = 4u,
  /* contiguous-prefix fast path for a compacted pool (the defragmentation
     plan of "The Integration Chasm", The Decision: Adapt the Kernel, Not the
     System): the caller guarantees that every request's prefix indices are
     consecutive, kv_indices[kv_indptr[b] + j] = kv_indices[kv_indptr[b]] + j
     for j < P_b (as mla_verify_compact leaves them).  The kernel then reads
     each request's first prefix index and gathers prefix key j from slot
     base_b + j; of the other prefix indices it reads only the last few
     (fewer than 64) before the tree keys.  A base outside the pool (or
     base_b + j past it) poisons the work items that gather those keys (NaN
     rows, MLA_VERIFY_DEVERR_SLOT_RANGE).  Prefixes that break the guarantee
     are not detected: their rows come from base_b + j (those last few from
     their own indices).  Tree keys (out_cache_loc) are read as usual. */
  MLA_VERIFY_FLAG_CONTIGUOUS_PREFIX = 8u
};

/* bits of the device error word (first uint32 of the workspace) */
enum {
  MLA_VERIFY_DEVERR_QO_INDPTR = 1u << 0,   /* qo_indptr decreasing, negative or past max_q_tokens */
  MLA_VERIFY_DEVERR_KV_INDPTR = 1u << 1,   /* kv_indptr decreasing, negative or past max_kv_tokens */
  MLA_VERIFY_DEVERR_TREE_SIZE = 1u << 2,   /* a request has more tree nodes than max_tree_nodes */
  MLA_VERIFY_DEVERR_MASK_INDPTR = 1u << 3, /* mask_indptr[b+1]-mask_indptr[b] != T_b*T_b (or
                                              T_b*(P_b+T_b) with full rows), or < 0 */
  MLA_VERIFY_DEVERR_SLOT_RANGE = 1u << 4,  /* a kv_indices / out_cache_loc entry outside [0, num_slots) */
  MLA_VERIFY_DEVERR_CAPACITY = 1u << 5,    /* work items exceeded the plan (internal bound) */
  MLA_VERIFY_DEVERR_MASK_PREFIX = 1u << 6  /* a prefix column of a full-row mask is zero (checked mode) */
};

/*
 * Plan-time bounds, host memory, filled by the caller.  Everything the launch
 * grid and the workspace size depend on is here; buffer contents may vary from
 * call to call (and from graph replay to replay) within these bounds.
 */
typedef struct {
  int32_t num_heads;           /* H >= 1 (head dims are fixed: 576 for Q.K^T, 512 for V) */
  int32_t max_batch;           /* bound on batch_size */
  int32_t max_q_tokens;        /* bound on sum_b T_b (= qo_indptr[B]) */
  int32_t max_tree_nodes;      /* bound on every T_b, 1..64 */
  int64_t max_kv_tokens;       /* bound on sum_b P_b (= kv_indptr[B]) */
  int32_t target_items;        /* key-range work items per call (about one per compute unit); 0 = auto */
  int32_t cu_count;            /* compute units of the target device; 0 = query the current device */
  int32_t kv_indices_dtype;    /* MLA_VERIFY_I32 or MLA_VERIFY_I64 */
  int32_t out_cache_loc_dtype; /* MLA_VERIFY_I64 or MLA_VERIFY_I32 */
  uint32_t flags;              /* MLA_VERIFY_FLAG_* */
  int32_t reserved[7];         /* must be zero */
} mla_verify_config_t;

/* An immutable plan value.  Opaque; copy freely; nothing to destroy. */
typedef struct {
  uint64_t opaque[64];
} mla_verify_plan_t;

/*
 * Per-call arguments.  Device pointers unless noted; strides in elements.
 *   q             bf16 [sum T, H, 576]: row (token t, head h) at
 *                 q + t*q_stride_tok + h*q_stride_head, 576 contiguous values;
 *                 16-byte aligned, strides multiples of 8.
 *   kv_pool       bf16 [num_slots, kv_row_stride], kv_row_stride >= 576 and a
 *                 multiple of 8, 16-byte aligned; num_slots < 2^31 and
 *                 kv_row_stride < 2^30 (MLA_VERIFY_ERR_UNSUPPORTED otherwise).
 *                 page_size = 1: slot s is one token's 576-wide latent row.
 *                 Without kv_new the rows of this call's draft tokens must
 *                 already be stored at out_cache_loc.
 *   qo_indptr     int32 [B+1], qo_indptr[0] = 0: request b owns query tokens
 *                 [qo_indptr[b], qo_indptr[b+1]), T_b of them, its tree nodes
 *                 in node order.
 *   kv_indptr     int32 [B+1]: request b's prefix is
 *                 kv_indices[kv_indptr[b] .. kv_indptr[b+1]), P_b = the difference.
 *   kv_indices    int32 or int64 (plan) [kv_indptr[B]]: pool slots of the prefix.
 *   out_cache_loc int64 or int32 (plan) [qo_indptr[B]]: pool slot of each tree node.
 *   custom_mask   uint8: request b's T_b x T_b block starts at mask_indptr[b],
 *                 row-major, row = query node i, column = key node k; nonzero
 *                 means node i sees node k.  No visibility is implied (a node
 *                 sees itself only if its diagonal entry is set).
 *   mask_indptr   int32 [B+1], mask_indptr[b+1] - mask_indptr[b] = T_b^2.
 *   out           fp32 [sum T, H, 512] at out + t*out_stride_tok + h*out_stride_head;
 *                 16-byte aligned, strides multiples of 4.
 *   lse           fp32 [sum T, H] at lse + t*lse_stride_tok + h, natural-log
 *                 log-sum-exp of the scaled visible scores; may be NULL.
 *   kv_new        bf16 [sum T, >= 576] at kv_new + t*kv_new_stride_tok, or NULL.
 *                 When given, the call first stores row t (576 values) into
 *                 the pool at slot out_cache_loc[t] (the KV save of this
 *                 step's draft tokens, fused into the call), then attends over
 *                 it, so the pool must be writable and those slots distinct
 *                 and fresh: none of them may appear in this call's
 *                 kv_indices.  Rows whose slot lies outside the pool are not
 *                 stored (the slot range error is raised as for any gathered
 *                 slot); with a metadata error nothing is stored.  16-byte
 *                 aligned, stride a multiple of 8.
 * A row that sees no key (P_b = 0 and an all-zero mask row) gets out = 0 and
 * lse = -inf.  Key order within a request is the prefix, then the tree nodes;
 * a slot listed twice is two keys.  Scores are sm_scale * (q . k), sm_scale
 * finite and positive (the softmax scale; anything else is an invalid
 * argument).
 */
typedef struct {
  int32_t batch_size;          /* B, 0..max_batch (host value, fixed at capture) */
  float sm_scale;
  const void* q;
  int64_t q_stride_tok;
  int64_t q_stride_head;
  const void* kv_pool;
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
  const void* kv_new;          /* optional: draft rows to store at out_cache_loc first */
  int64_t kv_new_stride_tok;
} mla_verify_args_t;

/* Where each workspace region lives (byte offsets from the workspace base,
   every offset 256-byte aligned) and the fixed launch shape of the plan. */
typedef struct {
  uint64_t total_bytes;
  uint64_t header_offset;     /* uint32 error word, int32 n_items, int32 total_q, int32 chunk_keys, int32 batch,
                                 int32 max_chunks (key ranges of the request with the most), uint32 metadata
                                 error bits */
  uint64_t request_offset;    /* int32 [max_batch][8]: P, T, q0, kv0, row_blocks, chunks, item_base, mask0 */
  uint64_t anc_offset;        /* uint64 [max_q_tokens]: packed tree visibility of each node */
  uint64_t items_offset;      /* int32 [item_capacity][8]: b, row_block, chunk, key0, key1, row0, nrows, 0 */
  uint64_t partial_o_offset;  /* fp32 [item_capacity][rows_per_item][512] unnormalised partial outputs */
  uint64_t partial_ml_offset; /* fp32 [item_capacity][rows_per_item][2] running max (log2 units) and sum */
  uint64_t trace_offset;      /* int64 [max_kv_tokens + max_q_tokens]: request b's key j at
                                 kv_indptr[b] + qo_indptr[b] + j, the index value it was gathered by;
                                 0 without the trace flag */
  uint64_t stats_offset;      /* mla_verify_compare_stats_t written by mla_verify_compare */
  uint64_t tokens_offset;     /* int32 [max_q_tokens][4]: per query token, its request's first token,
                                 first work item, row blocks and key ranges (read by the merge) */
  uint64_t errors_offset;     /* int32 [partial_grid]: device error bits found by each split-partial
                                 workgroup (folded into the error word by the merge) */
  int32_t item_capacity;
  int32_t rows_per_item;      /* query rows (token x head) per work item */
  int32_t keys_per_tile;      /* keys staged per inner-loop step */
  int32_t target_items;
  int32_t partial_grid;       /* workgroups of the split-partial launch */
  int32_t merge_grid;         /* workgroups of the merge launch */
} mla_verify_layout_t;

/* Validate a config and compute the plan: host arithmetic only (the one
   possible HIP call is the compute-unit query when cfg->cu_count == 0).  The
   plan fixes both launch grids, so that a captured call stays valid while the
   buffers' contents change between replays ("The Capture-Safe Kernel",
   Decision 3: a fixed split grid; Decision 6: buffers refreshed in place). */
mla_verify_status_t mla_verify_plan(const mla_verify_config_t* cfg, mla_verify_plan_t* plan);

/* Bytes of device workspace run() needs for this plan (256-byte aligned
   base).  The workspace holds the partial softmax statistics of the key
   ranges and the plan tables; the caller allocates it once and passes it to
   every call, so no call allocates ("The Capture-Safe Kernel", Decision 4). */
mla_verify_status_t mla_verify_workspace_size(const mla_verify_plan_t* plan, size_t* bytes);

/* Enqueue the verify attention on `stream` (a hipStream_t; NULL = the null
   stream): two kernel launches and nothing else - split partials (each
   workgroup derives the plan, prefix lengths and tree words from the raw
   metadata buffers on the device: "The Capture-Safe Kernel", Decisions 1, 2
   and 5) and the merge of the partial statistics (Decision 4).  It makes no
   allocation, host sync, host read of device data or temporary, so it may be
   recorded into a hipGraph ("The Capture-Safe Kernel", The Core Problem).
   workspace: device memory of at least workspace_size bytes, 256-byte
   aligned, owned by the caller; its previous contents are ignored.  Returns
   the first argument error found (nothing is enqueued then) or
   MLA_VERIFY_ERR_LAUNCH if HIP refuses a launch. */
mla_verify_status_t mla_verify_run(const mla_verify_plan_t* plan, const mla_verify_args_t* args,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* run() without a caller workspace, for callers that cannot allocate device
   memory (code under hipGraph capture, tight serving loops, harnesses that
   forbid allocation): the same two launches, with a workspace taken from a
   device array of MLA_VERIFY_STATIC_SCRATCH_BYTES that the library holds on
   each GPU it runs on until the process ends.  The array's address on the
   current device is looked up on the first call with that device current
   (make that first call outside capture); the stream must belong to the
   current device.  It calls no hipMalloc / hipFree.  All calls on one GPU
   share its array: calls that overlap on one GPU race, so serialise them
   (one stream, or events); the workspace-resident results (header error
   word, trace) of the last call live in that array, not in caller memory.
   Returns MLA_VERIFY_ERR_WORKSPACE_TOO_SMALL (before anything is enqueued)
   when the plan needs a larger workspace, the argument errors of run(), or
   MLA_VERIFY_ERR_LAUNCH when the array cannot be located or a launch fails. */
mla_verify_status_t mla_verify_run_static(const mla_verify_plan_t* plan, const mla_verify_args_t* args,
                                          void* stream);

/* One of run()'s two launches (phase 0 = split partials with the device-side
   plan, 1 = merge), with the same checks; run() == phases 0, 1 in order on
   one stream.  For per-kernel timing. */
mla_verify_status_t mla_verify_run_phase(const mla_verify_plan_t* plan, const mla_verify_args_t* args,
                                         void* workspace, size_t workspace_bytes, void* stream,
                                         int32_t phase);

/* Workspace regions and launch shape of a plan (host only). */
mla_verify_status_t mla_verify_workspace_layout(const mla_verify_plan_t* plan,
                                                mla_verify_layout_t* layout);

/* Static description of a status code. */
const char* mla_verify_status_string(mla_verify_status_t status);

/*
 * Shadow comparison ("The Launch Wrapper", The Design Decision: Three Modes of
 * Operation - the validate mode: the serving system keeps returning its own
 * attention result while this library's result is computed beside it and
 * compared).  After run() on the same stream, compare() checks
 * args->out / args->lse against the caller's reference, in the same layout,
 * over the call's query tokens, and accumulates into the workspace's stats
 * region (zeroed by every run()); read it after a sync.  One launch,
 * capture-safe.  ref_lse may be NULL.  An element counts as over when
 * |out - ref| > 2 bf16 ULP of ref (2^(floor(log2 |ref|) - 7), |ref| floored at
 * 2^-126) or exactly one of the two is NaN.
 */
typedef struct {
  uint32_t max_abs_diff_bits;  /* fp32 bits of max |out - ref| over pairs that are both finite */
  uint32_t count_over;         /* elements over the 2-ULP bound (NaN mismatches included) */
  uint32_t count_total;        /* elements compared */
  uint32_t max_lse_diff_bits;  /* fp32 bits of max |lse - ref_lse| over finite pairs */
  uint32_t count_nan_mismatch; /* out elements where exactly one of the two is NaN */
  uint32_t count_lse_mismatch; /* lse entries where exactly one of the two is finite */
  uint32_t reserved[2];
} mla_verify_compare_stats_t;

mla_verify_status_t mla_verify_compare(const mla_verify_plan_t* plan, const mla_verify_args_t* args,
                                       const float* ref_out, int64_t ref_out_stride_tok,
                                       int64_t ref_out_stride_head, const float* ref_lse,
                                       int64_t ref_lse_stride_tok, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Prefix compaction (KV defragmentation, the later phase planned in "The
 * Integration Chasm", The Decision: Adapt the Kernel, Not the System, and "The
 * Capture-Safe Kernel", The Context: A Long Road to Production; the pages give
 * no algorithm, this is the plainest one): request b's prefix rows (the slots
 * kv_indices[kv_indptr[b] + j], j < P_b) are copied to the contiguous slots
 * dst_start[b] + j, and those kv_indices entries are rewritten to the new
 * slots, in place.  Uses batch_size, kv_pool (writable), kv_row_stride,
 * num_slots, kv_indptr and kv_indices (writable, the plan's dtype) of args.
 *   dst_start    int64 [batch_size], device memory.
 *   error_word   int32, device memory, zeroed by the caller: a row whose old
 *                or new slot lies outside the pool, or a request whose indptrs
 *                are out of range, is left as it is and sets
 *                MLA_VERIFY_DEVERR_SLOT_RANGE / _KV_INDPTR here.
 * The destination slots must hold no row that any request still reads (they
 * are fresh slots from the caller's allocator); the old slots may be freed
 * once the call has run.  One launch whose grid depends on the plan only,
 * capture-safe; no workspace.
 */
mla_verify_status_t mla_verify_compact(const mla_verify_plan_t* plan, const mla_verify_args_t* args,
                                       const int64_t* dst_start, int32_t* error_word, void* stream);

/*
 * Measurement helper, outside the attention path: enqueues on `stream` one
 * launch of `blocks` workgroups of four waves; each wave runs `iters` rounds of
 * four independent bf16 16x16x32 MFMAs (4 x 16,384 flops per round), so one
 * call performs blocks x 4 x iters x 65,536 flops.  Timing it gives the dense
 * bf16 MFMA rate reached at the clock the GPU holds under load.
 *   out   float [blocks x 256], device memory: each thread's accumulator sum
 *         (exact, so linear in iters, for iters <= 4).
 * Returns MLA_VERIFY_ERR_INVALID_ARGUMENT for iters < 1, blocks < 1 or a null
 * or misaligned out, MLA_VERIFY_ERR_LAUNCH if HIP refuses the launch.
 */
mla_verify_status_t mla_verify_calibrate_mfma(int32_t iters, int32_t blocks, float* out, void* stream);

/*
 * Measurement helper, outside the attention path: enqueues on `stream` one
 * launch of `blocks` workgroups of 256 threads that read every byte of `buf`
 * once, in 16-byte units at a grid stride, and write one float per thread to
 * `out` (a checksum of the words it read).  Timing it gives the HBM read rate.
 *   buf    device memory, 16-byte aligned, `bytes` long (a multiple of 16).
 *   out    float [blocks x 256], device memory.
 * Returns MLA_VERIFY_ERR_INVALID_ARGUMENT for a null or misaligned pointer,
 * bytes < 16 or not a multiple of 16, or blocks < 1; MLA_VERIFY_ERR_LAUNCH if
 * HIP refuses the launch.
 */
mla_verify_status_t mla_verify_calibrate_read(const void* buf, int64_t bytes, int32_t blocks, float* out,
                                              void* stream);

/* MLA_VERIFY_ABI_VERSION of the built library. */
int32_t mla_verify_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_H_ */
