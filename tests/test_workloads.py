"""The seeded input generator: reproducible, structurally valid instances."""
import numpy as np

from workloads import gen


def test_seed_reproduces_bits():
    a = gen.config("p5632_t16")
    b = gen.config("p5632_t16")
    for f in ("q", "rows", "row_slots", "kv_indices", "out_cache_loc", "custom_mask"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = gen.config("p5632_t16", seed=7)
    assert not np.array_equal(a.q, c.q)


def test_structure_of_configs():
    for name in ("tiny", "p5632_t16", "p23040_t32"):
        inst = gen.config(name)
        spec = gen.CONFIGS[name]
        assert inst.prefix_lens == spec["prefix_lens"] and inst.tree_sizes == spec["tree_sizes"]
        assert inst.q.shape == (sum(spec["tree_sizes"]), spec["num_heads"], 576)
        used = np.concatenate([inst.kv_indices.astype(np.int64), inst.out_cache_loc])
        assert len(np.unique(used)) == len(used)
        assert used.min() >= 0 and used.max() < inst.num_slots
        for par in inst.parents:
            assert par[0] == -1 and all(0 <= p < i for i, p in enumerate(par) if i)
    assert gen.config("tiny").parents == [[-1, 0, 1, 2]]


def test_mask_is_ancestor_or_self():
    inst = gen.config("p23040_t32")
    t = inst.tree_sizes[0]
    m = inst.custom_mask.reshape(t, t)
    par = inst.parents[0]
    assert np.all(np.diag(m) == 1)
    for i in range(t):
        for k in range(t):
            # k is visible from i iff walking parents from i reaches k
            j, seen = i, False
            while j >= 0:
                seen |= (j == k)
                j = par[j]
            assert bool(m[i, k]) == seen


def test_outliers_and_poison():
    inst = gen.make_instance([1000], [8], 2, num_slots=4096, seed=3, outlier_frac=0.01)
    vals = (inst.rows.astype(np.uint32) << 16).view(np.float32)
    big = np.abs(vals[:1000]).max(axis=1)
    assert (big > 12).sum() >= 5        # 10 rows scaled by 8 show up as large rows
    pool = inst.dense_pool()
    unused = np.setdiff1d(np.arange(4096), inst.row_slots)
    assert np.all(pool[unused] == 0xFFFF)
    assert np.array_equal(pool[inst.row_slots], inst.rows)
    view = inst.pool_view()
    assert np.array_equal(view[inst.row_slots[:5]], inst.rows[:5])
    assert np.all(view[unused[:3]] == 0xFFFF)


def test_segmented_batch_fits_bounds():
    bounds = gen.SEGMENTED_BOUNDS
    for r in range(2):
        inst = gen.segmented(r)
        assert inst.batch == 8
        assert inst.total_q <= bounds["max_q_tokens"]
        assert inst.total_kv <= bounds["max_kv_tokens"]
        assert max(inst.tree_sizes) <= bounds["max_tree_nodes"]
        assert all(1000 <= p <= 185000 for p in inst.prefix_lens)
        assert int(inst.mask_indptr[-1]) == sum(t * t for t in inst.tree_sizes)


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], np.float32)
    bits = gen.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0]


def test_decode_shapes():
    """Decode workloads: one node per request that sees itself, prefixes in range."""
    for name, b, h in (("decode_b32_h16", 32, 16), ("decode_b64_h128", 64, 128)):
        spec = gen.CONFIGS[name]
        assert len(spec["prefix_lens"]) == b and spec["tree_sizes"] == [1] * b
        assert all(512 <= p <= 8192 for p in spec["prefix_lens"]) and spec["num_heads"] == h
    inst = gen.config("decode_b32_h16")
    assert np.array_equal(inst.custom_mask, np.ones(32, np.uint8))
    assert np.array_equal(np.asarray(inst.mask_indptr), np.arange(33))
    assert np.array_equal(np.asarray(inst.qo_indptr), np.arange(33))
