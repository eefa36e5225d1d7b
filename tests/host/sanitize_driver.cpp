// Host-side driver for the sanitizer build of the C-ABI (mla_verify_api.cpp):
// the kernel launches and the two HIP device queries are stubbed, so every
// entry point runs its argument checks and plan arithmetic on the host only.
// Built with g++ -fsanitize=address,undefined; any report ends the process
// with a failure.  Prints "ok" when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "mla_verify.h"
#include "mla_verify_internal.h"

static int g_partial = 0, g_merge = 0, g_compare = 0, g_compact = 0;
static mlav::KernelParams g_last;

namespace mlav {
int launch_partial(const KernelParams& p, const mla_verify_layout_t&, void*) { ++g_partial; g_last = p; return 0; }
int launch_merge(const KernelParams& p, const mla_verify_layout_t&, void*) { ++g_merge; g_last = p; return 0; }
int launch_compare(const KernelParams& p, const mla_verify_layout_t&, void*) { ++g_compare; g_last = p; return 0; }
int launch_compact(const KernelParams& p, const int64_t*, int32_t*, void*) { ++g_compact; g_last = p; return 0; }
}  // namespace mlav

// the one HIP query a plan may make (cu_count == 0): a 256-CU device
extern "C" hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

static mla_verify_config_t config(int h, int mb, int mq, int64_t mkv) {
  mla_verify_config_t c;
  memset(&c, 0, sizeof(c));
  c.num_heads = h;
  c.max_batch = mb;
  c.max_q_tokens = mq;
  c.max_tree_nodes = 64;
  c.max_kv_tokens = mkv;
  c.cu_count = 0;
  c.kv_indices_dtype = MLA_VERIFY_I32;
  c.out_cache_loc_dtype = MLA_VERIFY_I64;
  return c;
}

static mla_verify_args_t fake_args() {
  // aligned, never dereferenced addresses
  mla_verify_args_t a;
  memset(&a, 0, sizeof(a));
  uintptr_t base = (uintptr_t)1 << 40;
  const void** f[] = {&a.q, &a.kv_pool};
  for (int i = 0; i < 2; ++i) *f[i] = (const void*)(base + (uintptr_t)i * (1u << 30));
  a.qo_indptr = (const int32_t*)(base + 2 * ((uintptr_t)1 << 30));
  a.kv_indptr = (const int32_t*)(base + 3 * ((uintptr_t)1 << 30));
  a.kv_indices = (const void*)(base + 4 * ((uintptr_t)1 << 30));
  a.out_cache_loc = (const void*)(base + 5 * ((uintptr_t)1 << 30));
  a.custom_mask = (const uint8_t*)(base + 6 * ((uintptr_t)1 << 30));
  a.mask_indptr = (const int32_t*)(base + 7 * ((uintptr_t)1 << 30));
  a.out = (float*)(base + 8 * ((uintptr_t)1 << 30));
  a.lse = (float*)(base + 9 * ((uintptr_t)1 << 30));
  a.batch_size = 1;
  a.sm_scale = 0.0721687836f;
  a.q_stride_tok = 8 * 576;
  a.q_stride_head = 576;
  a.kv_row_stride = 576;
  a.num_slots = 1 << 20;
  a.out_stride_tok = 8 * 512;
  a.out_stride_head = 512;
  a.lse_stride_tok = 8;
  return a;
}

int main() {
  mla_verify_plan_t plan;
  // plan arithmetic over a spread of bounds, including extremes
  const int heads[] = {1, 8, 64, 128};
  const int64_t kvs[] = {0, 1, 91136, 1480000, 100000000};
  for (int h : heads)
    for (int64_t kv : kvs)
      for (int mb : {1, 8, 1024}) {
        mla_verify_config_t c = config(h, mb, 512, kv);
        mla_verify_status_t st = mla_verify_plan(&c, &plan);
        if (st != MLA_VERIFY_OK) {
          CHECK(st == MLA_VERIFY_ERR_UNSUPPORTED);
          continue;
        }
        size_t ws = 0;
        mla_verify_layout_t lay;
        CHECK(mla_verify_workspace_size(&plan, &ws) == MLA_VERIFY_OK);
        CHECK(mla_verify_workspace_layout(&plan, &lay) == MLA_VERIFY_OK);
        CHECK(lay.total_bytes == ws && ws % 256 == 0);
        const uint64_t offs[] = {lay.header_offset, lay.request_offset, lay.anc_offset, lay.items_offset,
                                 lay.partial_o_offset, lay.partial_ml_offset, lay.stats_offset,
                                 lay.tokens_offset, lay.errors_offset};
        for (uint64_t o : offs) CHECK(o % 256 == 0 && o < ws);
        CHECK(lay.partial_grid % 8 == 0 && lay.partial_grid >= 8);
        CHECK((lay.item_capacity + 7) / 8 <= 4 * (lay.partial_grid / 8));
        CHECK(lay.merge_grid == 512 * h);
        CHECK(lay.errors_offset + (uint64_t)lay.partial_grid * 4 <= ws);
      }
  // rejected configs
  {
    mla_verify_config_t c = config(8, 1, 16, 100);
    c.max_tree_nodes = 65;
    CHECK(mla_verify_plan(&c, &plan) == MLA_VERIFY_ERR_UNSUPPORTED);
    c = config(0, 1, 16, 100);
    CHECK(mla_verify_plan(&c, &plan) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
    c = config(8, 1, 16, 100);
    c.reserved[6] = 1;
    CHECK(mla_verify_plan(&c, &plan) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
    c = config(8, 1, 16, (int64_t)1 << 31);
    CHECK(mla_verify_plan(&c, &plan) == MLA_VERIFY_ERR_UNSUPPORTED);
    CHECK(mla_verify_plan(nullptr, &plan) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
  }
  // run / run_phase / compare / compact argument checks against a real plan
  mla_verify_config_t c = config(8, 8, 512, 1480000);
  CHECK(mla_verify_plan(&c, &plan) == MLA_VERIFY_OK);
  size_t ws = 0;
  CHECK(mla_verify_workspace_size(&plan, &ws) == MLA_VERIFY_OK);
  void* wsp = (void*)((uintptr_t)1 << 44);
  mla_verify_args_t a = fake_args();
  CHECK(mla_verify_run(&plan, &a, wsp, ws, nullptr) == MLA_VERIFY_OK);
  CHECK(g_partial == 1 && g_merge == 1);
  CHECK((uintptr_t)g_last.errs >= (uintptr_t)wsp && (uintptr_t)g_last.errs < (uintptr_t)wsp + ws);
  CHECK(g_last.num_heads == 8 && g_last.batch == 1 && g_last.trace == nullptr);
  CHECK(mla_verify_run(&plan, &a, wsp, ws - 1, nullptr) == MLA_VERIFY_ERR_WORKSPACE_TOO_SMALL);
  CHECK(mla_verify_run(&plan, &a, (void*)((uintptr_t)wsp + 64), ws, nullptr) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
  CHECK(mla_verify_run(&plan, nullptr, wsp, ws, nullptr) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
  CHECK(mla_verify_run_phase(&plan, &a, wsp, ws, nullptr, 0) == MLA_VERIFY_OK && g_partial == 2);
  CHECK(mla_verify_run_phase(&plan, &a, wsp, ws, nullptr, 1) == MLA_VERIFY_OK && g_merge == 2);
  CHECK(mla_verify_run_phase(&plan, &a, wsp, ws, nullptr, 2) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
  mla_verify_args_t b = a;
  b.batch_size = 9;
  CHECK(mla_verify_run(&plan, &b, wsp, ws, nullptr) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
  b = a;
  b.kv_row_stride = 500;
  CHECK(mla_verify_run(&plan, &b, wsp, ws, nullptr) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
  b = a;
  b.num_slots = (int64_t)1 << 32;
  CHECK(mla_verify_run(&plan, &b, wsp, ws, nullptr) == MLA_VERIFY_ERR_UNSUPPORTED);
  b = a;
  b.kv_new = (const void*)((uintptr_t)1 << 41);
  b.kv_new_stride_tok = 570;
  CHECK(mla_verify_run(&plan, &b, wsp, ws, nullptr) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
  b.kv_new_stride_tok = 576;
  CHECK(mla_verify_run(&plan, &b, wsp, ws, nullptr) == MLA_VERIFY_OK);
  b = a;
  b.sm_scale = 1.0f / 0.0f;
  CHECK(mla_verify_run(&plan, &b, wsp, ws, nullptr) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
  // the contiguous-prefix fast path is a plan option that the launches see
  {
    mla_verify_config_t cf = config(8, 8, 512, 1480000);
    cf.flags = MLA_VERIFY_FLAG_CONTIGUOUS_PREFIX;
    mla_verify_plan_t pf;
    CHECK(mla_verify_plan(&cf, &pf) == MLA_VERIFY_OK);
    size_t wsf = 0;
    CHECK(mla_verify_workspace_size(&pf, &wsf) == MLA_VERIFY_OK && wsf == ws);
    CHECK(mla_verify_run(&pf, &a, wsp, wsf, nullptr) == MLA_VERIFY_OK);
    CHECK((g_last.flags & MLA_VERIFY_FLAG_CONTIGUOUS_PREFIX) != 0);
    cf.flags = 0x100;
    CHECK(mla_verify_plan(&cf, &pf) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
  }
  const float* ref = (const float*)((uintptr_t)1 << 42);
  CHECK(mla_verify_compare(&plan, &a, ref, 8 * 512, 512, nullptr, 0, wsp, ws, nullptr) == MLA_VERIFY_OK);
  CHECK(mla_verify_compare(&plan, &a, ref, 8 * 512, 510, nullptr, 0, wsp, ws, nullptr) ==
        MLA_VERIFY_ERR_INVALID_ARGUMENT);
  const int64_t* dst = (const int64_t*)((uintptr_t)1 << 43);
  int32_t* errw = (int32_t*)((uintptr_t)1 << 43) + 64;
  CHECK(mla_verify_compact(&plan, &a, dst, errw, nullptr) == MLA_VERIFY_OK && g_compact == 1);
  CHECK(mla_verify_compact(&plan, &a, nullptr, errw, nullptr) == MLA_VERIFY_ERR_INVALID_ARGUMENT);
  // a plan value that is not a plan
  mla_verify_plan_t junk;
  memset(&junk, 0x5a, sizeof(junk));
  CHECK(mla_verify_run(&junk, &a, wsp, ws, nullptr) == MLA_VERIFY_ERR_BAD_PLAN);
  CHECK(mla_verify_workspace_size(&junk, &ws) == MLA_VERIFY_ERR_BAD_PLAN);
  for (int s = 0; s <= 6; ++s) CHECK(mla_verify_status_string((mla_verify_status_t)s) != nullptr);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
