"""Prefix compaction (KV defragmentation): rows move to contiguous fresh slots,
kv_indices is rewritten in place, and the verify call on the compacted pool
gives bit-identical results."""
import numpy as np
import pytest

from tests.gpu_helpers import assert_gate, need_gpu, oracle, say
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx64", [False, True])
def test_compaction_moves_rows_and_keeps_results(idx64):
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    inst = gen.make_instance([3000, 0, 129, 1700], [16, 3, 7, 5], 8, num_slots=16384, seed=98)
    say(f"compaction idx64={idx64}")
    di = DeviceInputs(inst, kv_indices_dtype=B.I64 if idx64 else B.I32)
    # fresh slots after the used pool, poisoned like every unused slot
    base = inst.num_slots + 32
    extra = torch.full((32 + inst.total_kv + 32, di.pool.shape[1]), -1, dtype=di.pool.dtype, device=di.pool.device)
    di.pool = torch.cat([di.pool, extra])
    di.num_slots = di.pool.shape[0]
    v = Verifier.for_inputs(di)
    out, lse = di.alloc_outputs()
    args = v.args(di, out, lse)
    B.run(v.plan, args, v.workspace)
    torch.cuda.synchronize()
    out0, lse0 = out.cpu().numpy().copy(), lse.cpu().numpy().copy()
    old = di.kv_indices.cpu().numpy().astype(np.int64)[:inst.total_kv]
    dst = torch.tensor([base + int(inst.kv_indptr[b]) for b in range(inst.batch)], dtype=torch.int64,
                       device=di.pool.device)
    err = torch.zeros(1, dtype=torch.int32, device=di.pool.device)
    B.compact(v.plan, args, dst, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    new = di.kv_indices.cpu().numpy().astype(np.int64)[:inst.total_kv]
    assert np.array_equal(new, base + np.arange(inst.total_kv))
    moved = di.pool[torch.from_numpy(new).to(di.pool.device)][:, :576].cpu().numpy().view(np.uint16)
    assert np.array_equal(moved, inst.pool_view()[old][:, :576])
    out.fill_(float("nan"))
    B.run(v.plan, args, v.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), out0.view(np.uint32))
    assert np.array_equal(lse.cpu().numpy().view(np.uint32), lse0.view(np.uint32))
    ref_out, ref_lse, _ = oracle(inst)
    assert_gate(out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, label="compacted")


def test_compaction_out_of_pool_destination_is_refused():
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    inst = gen.make_instance([500, 200], [4, 4], 8, num_slots=4096, seed=99)
    say("compaction out of pool")
    di = DeviceInputs(inst)
    extra = torch.full((600, di.pool.shape[1]), -1, dtype=di.pool.dtype, device=di.pool.device)
    di.pool = torch.cat([di.pool, extra])
    di.num_slots = di.pool.shape[0]
    v = Verifier.for_inputs(di)
    out, lse = di.alloc_outputs()
    args = v.args(di, out, lse)
    before = di.kv_indices.cpu().numpy().copy()
    # request 0 moves to fresh slots; request 1's range would run past the
    # pool end: its first 50 rows move, the rest stay where they are
    dst = torch.tensor([inst.num_slots, di.num_slots - 50], dtype=torch.int64, device=di.pool.device)
    err = torch.zeros(1, dtype=torch.int32, device=di.pool.device)
    B.compact(v.plan, args, dst, err)
    torch.cuda.synchronize()
    assert int(err.item()) == B.DEVERR_SLOT_RANGE
    after = di.kv_indices.cpu().numpy()
    k1 = int(inst.kv_indptr[1])
    assert np.array_equal(after[:k1], inst.num_slots + np.arange(k1))
    dst1 = di.num_slots - 50 + np.arange(inst.total_kv - k1)
    ok = dst1 < di.num_slots
    assert ok.sum() == 50
    assert np.array_equal(after[k1:inst.total_kv][ok], dst1[ok])
    assert np.array_equal(after[k1:inst.total_kv][~ok], before[k1:inst.total_kv][~ok])


@pytest.mark.parametrize("idx64", [False, True])
def test_contiguous_prefix_fast_path(idx64):
    """With MLA_VERIFY_FLAG_CONTIGUOUS_PREFIX on a compacted pool the call
    gathers prefix key j from kv_indices[kv0] + j: the same rows, so the same
    bits as the index path, and the prefix indices in the middle of a prefix
    are never read.  A base outside the pool poisons its request only."""
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    # prefixes: several slot blocks, none, shorter than a tile share, one
    # block plus a ragged tail, and one ending inside a 64-key share
    inst = gen.make_instance([3000, 0, 129, 1700, 40, 700], [16, 3, 7, 5, 2, 9], 8, num_slots=16384, seed=97)
    say(f"contiguous prefix idx64={idx64}")
    di = DeviceInputs(inst, kv_indices_dtype=B.I64 if idx64 else B.I32)
    base = inst.num_slots + 32
    extra = torch.full((32 + inst.total_kv + 32, di.pool.shape[1]), -1, dtype=di.pool.dtype, device=di.pool.device)
    di.pool = torch.cat([di.pool, extra])
    di.num_slots = di.pool.shape[0]
    flags = B.FLAG_TRACE_KEYS
    v = Verifier.for_inputs(di, flags=flags)
    vf = Verifier.for_inputs(di, flags=flags | B.FLAG_CONTIGUOUS_PREFIX)
    out, lse = di.alloc_outputs()
    args = v.args(di, out, lse)
    dst = torch.tensor([base + int(inst.kv_indptr[b]) for b in range(inst.batch)], dtype=torch.int64,
                       device=di.pool.device)
    err = torch.zeros(1, dtype=torch.int32, device=di.pool.device)
    B.compact(v.plan, args, dst, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    n_tr = inst.total_kv + inst.total_q

    def call(ver):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ver(di, out, lse)
        torch.cuda.synchronize()
        tr = ver.region(ver.layout.trace_offset, n_tr, torch.int64).cpu().numpy().copy()
        return out.cpu().numpy().copy(), lse.cpu().numpy().copy(), tr, ver.error_word()

    o_idx, l_idx, tr_idx, e_idx = call(v)
    o_fp, l_fp, tr_fp, e_fp = call(vf)
    assert e_idx == 0 and e_fp == 0
    assert np.array_equal(tr_fp, tr_idx)
    assert np.array_equal(o_fp.view(np.uint32), o_idx.view(np.uint32))
    assert np.array_equal(l_fp.view(np.uint32), l_idx.view(np.uint32))
    ref_out, ref_lse, _ = oracle(inst)
    assert_gate(o_fp, l_fp, ref_out, ref_lse, label="contiguous prefix")

    # indices in the middle of request 0's prefix and of request 3's are not
    # read: scrambling them changes nothing
    kvp = np.asarray(inst.kv_indptr, dtype=np.int64)
    saved = di.kv_indices.clone()
    for b, lo, hi in ((0, 300, 2800), (3, 1, 1500)):
        n = hi - lo
        junk = torch.randint(0, inst.num_slots, (n,), dtype=torch.int64, device=di.pool.device)
        di.kv_indices[int(kvp[b]) + lo:int(kvp[b]) + hi] = junk.to(di.kv_indices.dtype)
    o_s, l_s, tr_s, e_s = call(vf)
    assert e_s == 0
    assert np.array_equal(o_s.view(np.uint32), o_idx.view(np.uint32))
    assert np.array_equal(l_s.view(np.uint32), l_idx.view(np.uint32))
    assert np.array_equal(tr_s, tr_idx)

    # a base outside the pool (or, for 64-bit indices, with a high word set)
    # poisons request 2 alone
    di.kv_indices.copy_(saved)
    bad = (1 << 40) + int(dst[2].item()) if idx64 else di.num_slots + 5
    di.kv_indices[int(kvp[2])] = bad
    o_b, l_b, _, e_b = call(vf)
    assert e_b & B.DEVERR_SLOT_RANGE
    q = np.asarray(inst.qo_indptr, dtype=np.int64)
    rows2 = slice(int(q[2]), int(q[3]))
    assert np.isnan(o_b[rows2]).all() and np.isnan(l_b[rows2]).all()
    keep = np.ones(o_b.shape[0], dtype=bool)
    keep[rows2] = False
    assert np.array_equal(o_b[keep].view(np.uint32), o_idx[keep].view(np.uint32))
    assert np.array_equal(l_b[keep].view(np.uint32), l_idx[keep].view(np.uint32))


def _fast_path_case(name):
    """(device instance, oracle instance, DeviceInputs keywords, plan flags) of
    one fast-path case."""
    from speculative_decoding_mla_page_amd import binding as B
    from tests.test_gpu_mask_layout import full_row_instance
    rng = np.random.default_rng(500)
    if name in ("decode40", "decode100"):
        n = 40 if name == "decode40" else 100
        prefixes = rng.integers(0, 3000, n).tolist()
        prefixes[3] = 0
        inst = gen.make_instance(prefixes, [1] * n, 16, num_slots=1 << 19, seed=501 + n)
        return inst, inst, {}, 0
    mixed = gen.make_instance([0, 37, 1500, 1, 77, 2600], [3, 0, 16, 1, 5, 32], 8, num_slots=16384, seed=502)
    if name == "full_rows_checked":
        return full_row_instance(mixed), mixed, {}, B.FLAG_MASK_FULL_ROWS | B.FLAG_CHECK_PREFIX_MASK
    if name == "fused_save":
        return mixed, mixed, {"fused_save": True}, 0
    if name == "ocl_int32_kv_int64":
        return mixed, mixed, {"out_cache_loc_dtype": B.I32, "kv_indices_dtype": B.I64}, 0
    raise ValueError(name)


@pytest.mark.parametrize("name", ["decode40", "decode100", "full_rows_checked", "fused_save",
                                  "ocl_int32_kv_int64"])
def test_contiguous_prefix_matches_index_path(name):
    """The fast path gives the index path's bits on a compacted pool, with each
    plan option and with many requests (the multi-wave plan)."""
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    inst, ref_inst, dev_kw, flags = _fast_path_case(name)
    say(f"contiguous prefix vs index path: {name}")
    di = DeviceInputs(inst, **dev_kw)
    base = di.num_slots + 32
    extra = torch.full((32 + inst.total_kv + 32, di.pool.shape[1]), -1, dtype=di.pool.dtype, device=di.pool.device)
    di.pool = torch.cat([di.pool, extra])
    di.num_slots = di.pool.shape[0]
    tn = max(1, max(int(t) for t in inst.tree_sizes))
    v = Verifier.for_inputs(di, flags=flags, max_tree_nodes=tn)
    vf = Verifier.for_inputs(di, flags=flags | B.FLAG_CONTIGUOUS_PREFIX, max_tree_nodes=tn)
    out, lse = di.alloc_outputs()
    dst = torch.tensor([base + int(inst.kv_indptr[b]) for b in range(inst.batch)], dtype=torch.int64,
                       device=di.pool.device)
    err = torch.zeros(1, dtype=torch.int32, device=di.pool.device)
    B.compact(v.plan, v.args(di, out, lse), dst, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    res = []
    for ver in (v, vf):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ver(di, out, lse)
        torch.cuda.synchronize()
        assert ver.error_word() == 0
        res.append((out.cpu().numpy().copy(), lse.cpu().numpy().copy()))
    (o_i, l_i), (o_f, l_f) = res
    assert np.array_equal(o_f.view(np.uint32), o_i.view(np.uint32))
    assert np.array_equal(l_f.view(np.uint32), l_i.view(np.uint32))
    ref_out, ref_lse, _ = oracle(ref_inst)
    assert_gate(o_f, l_f, ref_out, ref_lse, label=f"contiguous prefix {name}")
