"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: gathered keys, tree-visibility words and work items bit-exact; outputs
within max-abs 1e-2 with >= 99.9% of elements within 2 bf16 ULP of the
oracle; LSE within 1e-3.
"""
import numpy as np
import pytest

from workloads import gen
from tests.gpu_helpers import assert_gate, assert_rows_finite, need_gpu, oracle, oracle_blocked, run_gpu, say

pytestmark = pytest.mark.gpu


def _check_metadata(inst, v, rec):
    """Tree words, gathered keys (trace), the work-item table, the request
    table and the merge's token entries, bit for bit."""
    import torch
    lay = v.layout
    total_q, total_kv = inst.total_q, inst.total_kv
    hdr = v.header()
    assert hdr[0] == 0, f"device error word {hdr[0]:#x}"
    n_items = int(hdr[1])
    assert int(hdr[2]) == total_q
    anc = v.region(lay.anc_offset, max(total_q, 1), torch.int64).cpu().numpy().view(np.uint64)
    assert np.array_equal(anc[:total_q], rec["anc"])
    if lay.trace_offset:
        tr = v.region(lay.trace_offset, total_kv + total_q, torch.int64).cpu().numpy()
        for b in range(inst.batch):
            if inst.tree_sizes[b] == 0:
                continue            # no query rows: nothing is gathered for this request
            base = int(inst.kv_indptr[b]) + int(inst.qo_indptr[b])
            keys = rec["keys"][b]
            assert np.array_equal(tr[base:base + len(keys)], keys), f"request {b}"
    items = v.region(lay.items_offset, max(n_items, 1) * 8, torch.int32).cpu().numpy().reshape(-1, 8)
    items = items[:n_items]
    rows_per = lay.rows_per_item
    for b in range(inst.batch):
        t_b = inst.tree_sizes[b]
        n_b = inst.prefix_lens[b] + t_b
        mine = items[items[:, 0] == b]
        n_rb = (t_b * inst.num_heads + rows_per - 1) // rows_per
        assert len(set(mine[:, 1].tolist())) == n_rb
        for rb in range(n_rb):
            blk = mine[mine[:, 1] == rb]
            cover = np.zeros(n_b, np.int32)
            for e in blk:
                assert e[5] == rb * rows_per
                assert e[6] == min(rows_per, t_b * inst.num_heads - rb * rows_per)
                cover[e[3]:e[4]] += 1
            assert np.all(cover == 1), f"request {b} row block {rb} keys not covered exactly once"
    # the request table and the merge's per-token entries agree with the
    # item table
    req = v.region(lay.request_offset, max(inst.batch, 1) * 8, torch.int32).cpu().numpy().reshape(-1, 8)
    chunks = [int(req[b][5]) for b in range(inst.batch)]
    assert int(hdr[5]) == max(chunks + [0]), "max_chunks in the header"
    tok = v.region(lay.tokens_offset, max(total_q, 1) * 4, torch.int32).cpu().numpy().reshape(-1, 4)
    for b in range(inst.batch):
        for t in range(int(inst.qo_indptr[b]), int(inst.qo_indptr[b + 1])):
            assert tok[t].tolist() == [int(inst.qo_indptr[b]), int(req[b][6]), int(req[b][4]), chunks[b]], f"token {t}"
    for b in range(inst.batch):
        mine = np.nonzero(items[:, 0] == b)[0]
        if len(mine):
            assert int(mine.min()) == int(req[b][6]) and len(mine) == int(req[b][4]) * chunks[b]
    # every workgroup's error slot is written (zero on a clean call)
    errs = v.region(lay.errors_offset, lay.partial_grid, torch.int32).cpu().numpy()
    assert np.all(errs == 0), "error slots"


@pytest.mark.parametrize("name", ["tiny", "p5632_t16", "p23040_t32", "p91136_t32"])
def test_config_parity_full(name):
    need_gpu()
    inst = gen.config(name)
    say(f"config {name}: P={inst.prefix_lens} T={inst.tree_sizes} H={inst.num_heads}")
    from speculative_decoding_mla_page_amd import binding as B
    out, lse, v, _ = run_gpu(inst, flags=B.FLAG_TRACE_KEYS)
    ref_out, ref_lse, rec = oracle(inst)
    _check_metadata(inst, v, rec)
    assert_gate(out, lse, ref_out, ref_lse, label=name)


def test_many_key_ranges_per_row():
    """One row block over a 40k-key prefix: about 250 key ranges per query row,
    so the merge folds its partials over several passes of every wave."""
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = gen.make_instance([40000], [6], 8, num_slots=65536, seed=97)
    say("many key ranges: P=40000 T=6 H=8")
    out, lse, v, _ = run_gpu(inst, flags=B.FLAG_TRACE_KEYS)
    assert int(v.header()[5]) > 128, "expected more key ranges than one pass of eight waves covers"
    ref_out, ref_lse, rec = oracle(inst)
    _check_metadata(inst, v, rec)
    assert_gate(out, lse, ref_out, ref_lse, label="many-ranges")


@pytest.mark.parametrize("max_nodes,prefixes,trees", [
    (1, [700, 1500, 33, 4000], [1, 1, 1, 1]),      # 8 rows per request: one row tile
    (2, [700, 1500, 0, 129], [2, 1, 2, 2]),        # up to 16 rows: one row tile
    (4, [256, 3000, 77], [4, 3, 4]),               # up to 32 rows: two row tiles
])
def test_small_tree_plans(max_nodes, prefixes, trees):
    """Plans whose tree-size bound keeps every item under 64 rows run the
    split-partial instantiation without the empty row tiles' PV work."""
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = gen.make_instance(prefixes, trees, 8, num_slots=16384, seed=90 + max_nodes)
    say(f"small tree plan: max_tree_nodes={max_nodes} P={prefixes} T={trees}")
    out, lse, v, _ = run_gpu(inst, flags=B.FLAG_TRACE_KEYS, max_tree_nodes=max_nodes)
    ref_out, ref_lse, rec = oracle(inst)
    _check_metadata(inst, v, rec)
    assert_gate(out, lse, ref_out, ref_lse, label=f"max_tree_nodes={max_nodes}")


def test_config_parity_h64_full():
    """H = 64 (2,048 query rows): every row against the oracle (computed four
    tokens at a time), gathered keys and tree words bit-exact."""
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = gen.config("p91136_t32_h64")
    say("config p91136_t32_h64 (all 32 nodes x 64 heads)")
    out, lse, v, _ = run_gpu(inst, flags=B.FLAG_TRACE_KEYS)
    assert_rows_finite(out, lse, label="h64")
    ref_out, ref_lse, rec = oracle_blocked(inst, block_tokens=4)
    _check_metadata(inst, v, rec)
    assert_gate(out, lse, ref_out, ref_lse, label="p91136_t32_h64")


def test_mixed_batch_edges():
    """Empty tree, empty prefix, 64-node tree, 1-node tree, ragged tails, and
    rows that see no key at all (no prefix, empty mask row)."""
    need_gpu()
    inst = gen.make_instance([0, 37, 5000, 1, 77], [3, 0, 64, 1, 5], 8, num_slots=16384, seed=91)
    rng = np.random.default_rng(1)
    blocks = [np.asarray(inst.custom_mask[inst.mask_indptr[b]:inst.mask_indptr[b + 1]]).copy()
              for b in range(inst.batch)]
    blocks[0] = (rng.random(9) < 0.5).astype(np.uint8)
    blocks[0][3:6] = 0                          # node 1 of request 0 sees nothing
    blocks[4] = (rng.random(25) < 0.5).astype(np.uint8)   # arbitrary, asymmetric
    inst.custom_mask = np.concatenate(blocks)
    say("mixed batch")
    from speculative_decoding_mla_page_amd import binding as B
    out, lse, v, _ = run_gpu(inst, flags=B.FLAG_TRACE_KEYS)
    ref_out, ref_lse, rec = oracle(inst)
    _check_metadata(inst, v, rec)
    assert np.all(out[1] == 0) and np.all(lse[1] == -np.inf)
    assert_gate(out, lse, ref_out, ref_lse, label="mixed")


@pytest.mark.parametrize("label,batch,tree_hi,heads", [
    ("batch100", 100, 16, 8),      # more requests than one wave holds: the multi-wave plan
    ("decode300", 300, 1, 16),     # 300 one-node requests: several rounds, every candidate timed
])
def test_large_batch_plans(label, batch, tree_hi, heads):
    """Batches of more than 64 requests take the plan's multi-wave path (every
    thread takes requests, wave reductions and barriers); the second case has
    more items than one round holds, so every candidate length is timed."""
    need_gpu()
    rng = np.random.default_rng(400 + batch)
    prefixes = [int(x) for x in rng.integers(0, 3000, batch)]
    trees = [int(x) for x in rng.integers(1, tree_hi + 1, batch)]
    prefixes[3] = 0                             # one request with no prefix
    inst = gen.make_instance(prefixes, trees, heads, num_slots=1 << 19, seed=401 + batch)
    say(f"{label}: B={batch} keys={sum(prefixes) + sum(trees)} H={heads}")
    from speculative_decoding_mla_page_amd import binding as B
    out, lse, v, _ = run_gpu(inst, flags=B.FLAG_TRACE_KEYS, max_tree_nodes=max(trees))
    ref_out, ref_lse, rec = oracle(inst)
    _check_metadata(inst, v, rec)
    assert_rows_finite(out, lse, label=label)
    assert_gate(out, lse, ref_out, ref_lse, label=label)


def test_index_dtypes_strides_and_padded_rows():
    """int64 kv_indices, int32 out_cache_loc, strided q/out, pool rows of 640."""
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = gen.make_instance([3000, 129], [16, 7], 8, num_slots=8192, seed=92)
    say("dtypes/strides")
    out, lse, v, di = run_gpu(inst, kv_indices_dtype=B.I64, out_cache_loc_dtype=B.I32,
                              row_stride=640, q_pad_heads=3, out_pad_heads=2)
    assert not di.q.is_contiguous() and di.pool.stride(0) == 640
    ref_out, ref_lse, _ = oracle(inst)
    assert_gate(out, lse, ref_out, ref_lse, label="dtypes")


def test_duplicate_slots():
    need_gpu()
    inst = gen.make_instance([700], [9], 8, num_slots=4096, seed=93)
    inst.kv_indices[100:200] = inst.kv_indices[0:100]
    say("duplicate slots")
    out, lse, _, _ = run_gpu(inst)
    ref_out, ref_lse, _ = oracle(inst)
    assert_gate(out, lse, ref_out, ref_lse, label="dup")


def test_split_counts_agree():
    """The number of key ranges changes only rounding: 1 range vs many."""
    need_gpu()
    inst = gen.make_instance([9000], [12], 8, num_slots=16384, seed=94)
    ref_out, ref_lse, _ = oracle(inst)
    for target in (1, 7, 64, 1024):
        say(f"target_items {target}")
        out, lse, _, _ = run_gpu(inst, target_items=target)
        assert_gate(out, lse, ref_out, ref_lse, label=f"target{target}")


def test_slot_permutation_and_rerun_are_bit_identical():
    need_gpu()
    inst = gen.make_instance([4000, 333], [20, 6], 8, num_slots=16384, seed=95)
    say("permutation invariance")
    out1, lse1, v, di = run_gpu(inst)
    import torch
    out_b, lse_b = di.alloc_outputs()
    v(di, out_b, lse_b)
    torch.cuda.synchronize()
    assert np.array_equal(out1, out_b.cpu().numpy()) and np.array_equal(lse1, lse_b.cpu().numpy())
    perm = np.random.default_rng(4).permutation(inst.num_slots)
    inst.row_slots = perm[inst.row_slots]
    inst.kv_indices = perm[inst.kv_indices].astype(np.int32)
    inst.out_cache_loc = perm[inst.out_cache_loc].astype(np.int64)
    out2, lse2, _, _ = run_gpu(inst)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_single_node_and_chain_trees():
    need_gpu()
    for name, inst in [
        ("single", gen.make_instance([2500], [1], 8, num_slots=4096, seed=96)),
        ("chain", gen.make_instance([2500], [24], 8, num_slots=4096, seed=97, tree="chain")),
    ]:
        say(name)
        out, lse, _, _ = run_gpu(inst)
        ref_out, ref_lse, _ = oracle(inst)
        assert_gate(out, lse, ref_out, ref_lse, label=name)


def test_empty_batch_writes_nothing():
    need_gpu()
    import torch
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    inst = gen.make_instance([100], [4], 8, num_slots=1024, seed=98)
    di = DeviceInputs(inst)
    v = Verifier.for_inputs(di)
    out, lse = di.alloc_outputs()
    say("empty batch")
    v(di, out, lse, batch_size=0)
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all()
    assert v.error_word() == 0 and int(v.header()[1]) == 0


# ------------------------------------------------------------------ device errors
def test_slot_out_of_range_sets_error_and_nan_rows():
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = gen.make_instance([300, 200], [4, 3], 8, num_slots=2048, seed=99)
    inst.kv_indices[17] = 2048 + 5            # request 0 only
    say("slot out of range")
    out, lse, v, _ = run_gpu(inst)
    assert v.error_word() & B.DEVERR_SLOT_RANGE
    assert np.isnan(out[:4]).all() and np.isnan(lse[:4]).all()
    ref_out, ref_lse, _ = oracle(inst, tokens=[4, 5, 6])
    assert_gate(out, lse, ref_out, ref_lse, tokens=[4, 5, 6], label="other request")


def test_ranges_of_bad_slots_only_give_nan_rows():
    """Every prefix index of request 0 outside the pool: its all-prefix key
    ranges read slot 0, a NaN row here, so all their scores are NaN and their
    reference max stays -inf.  The poison must still reach the merged rows."""
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    inst = gen.make_instance([700, 200], [4, 3], 8, num_slots=2048, seed=103)
    used = set(np.asarray(inst.kv_indices).tolist()) | set(np.asarray(inst.out_cache_loc).tolist())
    assert 0 not in used
    inst.kv_indices = np.asarray(inst.kv_indices).copy()
    inst.kv_indices[:700] = 2048 + 5
    say("ranges of bad slots only")
    di = DeviceInputs(inst)
    di.pool[0] = -1                          # bf16 NaN bits
    v = Verifier.for_inputs(di)
    out, lse = di.alloc_outputs()
    v(di, out, lse)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert v.error_word() & B.DEVERR_SLOT_RANGE
    assert np.isnan(out[:4]).all() and np.isnan(lse[:4]).all()
    ref_out, ref_lse, _ = oracle(inst, tokens=[4, 5, 6])
    assert_gate(out, lse, ref_out, ref_lse, tokens=[4, 5, 6], label="other request")


@pytest.mark.parametrize("what", ["mask_indptr", "tree_size", "kv_indptr"])
def test_bad_metadata_sets_error_and_nan(what):
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = gen.make_instance([300, 200], [4, 9], 8, num_slots=2048, seed=100)
    kw = {}
    bit = None
    if what == "mask_indptr":
        inst.mask_indptr = inst.mask_indptr.copy()
        inst.mask_indptr[1] += 1
        bit = B.DEVERR_MASK_INDPTR
    elif what == "tree_size":
        kw["max_tree_nodes"] = 8
        bit = B.DEVERR_TREE_SIZE
    else:
        inst.kv_indptr = inst.kv_indptr.copy()
        inst.kv_indptr[1] = 600                 # request 1: prefix of -100
        bit = B.DEVERR_KV_INDPTR
    say(f"bad metadata {what}")
    out, lse, v, _ = run_gpu(inst, **kw)
    assert v.error_word() & bit
    assert np.isnan(out).all() and np.isnan(lse).all()
