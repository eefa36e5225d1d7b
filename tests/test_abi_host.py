"""C-ABI boundary checks that need no GPU: exports, struct layout, plan arithmetic,
host-side argument errors.  No call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

from speculative_decoding_mla_page_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_verify.h")


def _declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mla_verify_\w+)\s*\(", src, re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = B.lib()
    names = _declared_functions()
    assert {"mla_verify_plan", "mla_verify_workspace_size", "mla_verify_run"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mla_verify_abi_version() == B.ABI_VERSION == 7


def test_struct_layout_matches_header(tmp_path):
    """Compile a probe of the header with gcc and compare sizes/offsets with the ctypes mirror."""
    probe = tmp_path / "probe.c"
    fields = {"mla_verify_config_t": B.Config, "mla_verify_args_t": B.Args,
              "mla_verify_layout_t": B.Layout, "mla_verify_plan_t": B.Plan,
              "mla_verify_compare_stats_t": B.CompareStats}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "mla_verify.h"', 'int main(void){']
    for cname, py in fields.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0;}")
    probe.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(probe), "-o", str(exe)],
                   check=True)
    got = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    for line in filter(None, got):
        cname, fname, val = line.split()
        py = fields[cname]
        if fname == "size":
            assert ctypes.sizeof(py) == int(val), line
        else:
            assert getattr(py, fname).offset == int(val), line


def _plan(**kw):
    base = dict(num_heads=8, max_batch=8, max_q_tokens=512, max_kv_tokens=1_480_000, cu_count=256)
    base.update(kw)
    return B.plan(B.make_config(**base))


def test_plan_layout_arithmetic():
    p = _plan()
    lay = B.layout(p)
    rows = lay.rows_per_item
    assert rows in (64, 128) and lay.keys_per_tile == 32 and lay.target_items == 256
    # one partly filled key range per row block, at most
    assert lay.item_capacity == 2 * 256 + (512 * 8 + rows - 1) // rows + 8
    # about one split-partial workgroup per target item, in groups of 8, and
    # enough that none runs more than 4 items
    assert lay.partial_grid % 8 == 0 and lay.partial_grid >= 256
    assert (lay.item_capacity + 7) // 8 <= 4 * (lay.partial_grid // 8)
    wide = B.layout(_plan(target_items=8, num_heads=128, max_q_tokens=512))
    assert (wide.item_capacity + 7) // 8 <= 4 * (wide.partial_grid // 8) and wide.partial_grid > 8
    assert lay.merge_grid == 512 * 8
    offs = [lay.header_offset, lay.request_offset, lay.anc_offset, lay.items_offset,
            lay.partial_o_offset, lay.partial_ml_offset]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    assert lay.partial_ml_offset - lay.partial_o_offset >= lay.item_capacity * rows * 512 * 4
    assert lay.total_bytes >= lay.partial_ml_offset + lay.item_capacity * rows * 8
    assert B.workspace_size(p) == lay.total_bytes
    assert lay.trace_offset == 0
    # the small regions after the partials: comparison stats, the merge's
    # token entries, one error slot per split-partial workgroup (last)
    assert lay.stats_offset % 256 == 0 and lay.stats_offset >= lay.partial_ml_offset + lay.item_capacity * rows * 8
    assert lay.tokens_offset % 256 == 0 and lay.tokens_offset >= lay.stats_offset + ctypes.sizeof(B.CompareStats)
    assert lay.errors_offset % 256 == 0 and lay.errors_offset >= lay.tokens_offset + 512 * 16
    assert lay.total_bytes == lay.errors_offset + (lay.partial_grid * 4 + 255) // 256 * 256
    # no per-key region without the trace: the workspace does not grow with the prefix bound
    assert B.layout(_plan(max_kv_tokens=10)).total_bytes == lay.total_bytes
    t = B.layout(_plan(flags=B.FLAG_TRACE_KEYS))
    assert t.trace_offset % 256 == 0 and t.total_bytes >= t.trace_offset + (1_480_000 + 512) * 8
    # explicit target overrides the CU count
    assert B.layout(_plan(target_items=64)).target_items == 64


def test_plan_is_a_plain_value():
    p = _plan()
    q = B.Plan()
    ctypes.memmove(ctypes.byref(q), ctypes.byref(p), ctypes.sizeof(p))
    assert B.workspace_size(q) == B.workspace_size(p)


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=0), B.ERR_INVALID_ARGUMENT),
    (dict(max_batch=0), B.ERR_INVALID_ARGUMENT),
    (dict(max_q_tokens=0), B.ERR_INVALID_ARGUMENT),
    (dict(max_tree_nodes=65), B.ERR_UNSUPPORTED),
    (dict(max_tree_nodes=0), B.ERR_INVALID_ARGUMENT),
    (dict(max_batch=4096), B.ERR_UNSUPPORTED),
    (dict(kv_indices_dtype=7), B.ERR_INVALID_ARGUMENT),
    (dict(flags=0x80), B.ERR_INVALID_ARGUMENT),
    (dict(flags=B.FLAG_CHECK_PREFIX_MASK), B.ERR_INVALID_ARGUMENT),   # needs full mask rows
    (dict(max_kv_tokens=-1), B.ERR_INVALID_ARGUMENT),
    (dict(max_kv_tokens=2 ** 31), B.ERR_UNSUPPORTED),
])
def test_plan_rejects_bad_configs(kw, status):
    with pytest.raises(B.MlaVerifyError) as e:
        _plan(**kw)
    assert e.value.status == status


def test_reserved_fields_must_be_zero():
    c = B.make_config(8, 1, 4, 100, cu_count=4)
    c.reserved[3] = 1
    with pytest.raises(B.MlaVerifyError) as e:
        B.plan(c)
    assert e.value.status == B.ERR_INVALID_ARGUMENT


def test_garbage_plan_is_rejected():
    bogus = B.Plan()
    n = ctypes.c_size_t()
    assert B.lib().mla_verify_workspace_size(ctypes.byref(bogus), ctypes.byref(n)) == B.ERR_BAD_PLAN
    assert B.lib().mla_verify_run(ctypes.byref(bogus), None, None, 0, None) == B.ERR_BAD_PLAN


def _fake_args(**kw):
    """Argument struct with fake (never dereferenced) aligned addresses."""
    a = B.Args()
    a.batch_size = 1
    a.sm_scale = 0.07
    base = 1 << 40
    for i, f in enumerate(["q", "kv_pool", "qo_indptr", "kv_indptr", "kv_indices", "out_cache_loc",
                           "custom_mask", "mask_indptr", "out", "lse"]):
        setattr(a, f, base + i * (1 << 30))
    a.q_stride_tok, a.q_stride_head = 8 * 576, 576
    a.kv_row_stride, a.num_slots = 576, 1024
    a.out_stride_tok, a.out_stride_head = 8 * 512, 512
    a.lse_stride_tok = 8
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), B.ERR_INVALID_ARGUMENT),
    (dict(kv_pool=(1 << 40) + 8), B.ERR_INVALID_ARGUMENT),
    (dict(q_stride_head=577), B.ERR_INVALID_ARGUMENT),
    (dict(kv_row_stride=512), B.ERR_INVALID_ARGUMENT),
    (dict(num_slots=0), B.ERR_INVALID_ARGUMENT),
    (dict(out_stride_head=510), B.ERR_INVALID_ARGUMENT),
    (dict(batch_size=9), B.ERR_INVALID_ARGUMENT),
    (dict(batch_size=-1), B.ERR_INVALID_ARGUMENT),
    (dict(sm_scale=float("nan")), B.ERR_INVALID_ARGUMENT),
    (dict(sm_scale=0.0), B.ERR_INVALID_ARGUMENT),
    (dict(sm_scale=-0.07), B.ERR_INVALID_ARGUMENT),
])
def test_run_rejects_bad_arguments_before_launch(kw, status):
    p = _plan()
    a = _fake_args(**kw)
    ws = 1 << 44
    st = B.lib().mla_verify_run(ctypes.byref(p), ctypes.byref(a), ws, B.workspace_size(p), None)
    assert st == status


def test_run_rejects_small_or_misaligned_workspace():
    p = _plan()
    a = _fake_args()
    need = B.workspace_size(p)
    lib = B.lib()
    assert lib.mla_verify_run(ctypes.byref(p), ctypes.byref(a), 1 << 44, need - 1, None) == \
        B.ERR_WORKSPACE_TOO_SMALL
    assert lib.mla_verify_run(ctypes.byref(p), ctypes.byref(a), (1 << 44) + 128, need, None) == \
        B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_run(ctypes.byref(p), ctypes.byref(a), None, need, None) == \
        B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_run_phase(ctypes.byref(p), ctypes.byref(a), 1 << 44, need, None, 2) == \
        B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_run_phase(ctypes.byref(p), ctypes.byref(a), 1 << 44, need, None, -1) == \
        B.ERR_INVALID_ARGUMENT


def test_run_static_rejects_before_any_hip_call():
    """The allocation-free entry point checks the plan size and the arguments
    on the host first (no GPU needed for these answers)."""
    lib = B.lib()
    big = B.plan(B.make_config(128, 64, 4096, 1_000_000, cu_count=256))
    assert B.workspace_size(big) > B.STATIC_SCRATCH_BYTES
    assert lib.mla_verify_run_static(ctypes.byref(big), ctypes.byref(_fake_args()), None) == \
        B.ERR_WORKSPACE_TOO_SMALL
    assert lib.mla_verify_run_static(ctypes.byref(B.Plan()), None, None) == B.ERR_BAD_PLAN
    p = _plan(max_kv_tokens=100_000)
    assert B.workspace_size(p) <= B.STATIC_SCRATCH_BYTES
    assert lib.mla_verify_run_static(ctypes.byref(p), ctypes.byref(_fake_args(q=0)), None) == \
        B.ERR_INVALID_ARGUMENT


def test_calibrate_mfma_rejects_bad_arguments_before_launch():
    lib = B.lib()
    assert lib.mla_verify_calibrate_mfma(0, 1, 1 << 44, None) == B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_calibrate_mfma(1, 0, 1 << 44, None) == B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_calibrate_mfma(1, 1, None, None) == B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_calibrate_mfma(1, 1, (1 << 44) + 2, None) == B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_calibrate_read(None, 1024, 1, 1 << 44, None) == B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_calibrate_read(1 << 44, 1000, 1, 1 << 44, None) == B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_calibrate_read((1 << 44) + 8, 1024, 1, 1 << 44, None) == B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_calibrate_read(1 << 44, 1024, 0, 1 << 44, None) == B.ERR_INVALID_ARGUMENT
    assert lib.mla_verify_calibrate_read(1 << 44, 1024, 1, None, None) == B.ERR_INVALID_ARGUMENT


def test_status_strings():
    assert B.status_string(B.OK) == "ok"
    assert "workspace" in B.status_string(B.ERR_WORKSPACE_TOO_SMALL)


def test_mask_layout_flags_plan():
    """Full-row masks and the prefix check are plan options that change no region."""
    lay = B.layout(_plan(flags=B.FLAG_MASK_FULL_ROWS | B.FLAG_CHECK_PREFIX_MASK))
    base = B.layout(_plan())
    assert lay.total_bytes == base.total_bytes and lay.errors_offset == base.errors_offset


def test_contiguous_prefix_flag_plan():
    """The contiguous-prefix fast path is a plan option that changes no region."""
    lay = B.layout(_plan(flags=B.FLAG_CONTIGUOUS_PREFIX))
    base = B.layout(_plan())
    assert lay.total_bytes == base.total_bytes and lay.partial_grid == base.partial_grid
