"""A longer seeded random sweep of the whole call against the oracle, run by hand on a
machine with the GPU (python tests/random_sweep.py [cases]); pytest does not collect it.  Each case
draws batch (up to 200), heads (1 to 128, including ones that do not divide 64), prefix
and tree lengths, mask layout and prefix check, the fused save, index dtypes, pool row
stride, work-item target, and the contiguous-prefix fast path on a compacted pool.  It
stops at the first case outside the gate."""
import os, sys, time
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import numpy as np, torch
from speculative_decoding_mla_page_amd import binding as B
from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
from workloads import gen
from tests.gpu_helpers import gate_stats, oracle
from tests.test_gpu_mask_layout import full_row_instance

N = int(sys.argv[1]) if len(sys.argv) > 1 else 100
MAX_WORK = 30_000_000
t_start = time.time()
for case in range(N):
    seed = 50_000 + case
    rng = np.random.default_rng(seed)
    heads = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 20, 32, 40, 64, 100, 128]))
    batch = int(rng.choice([1, 2, 5, 17, 40, 64, 65, 100, 200]))
    while True:
        kind = rng.random(batch)
        prefixes = np.where(kind < 0.1, 0, np.where(kind < 0.6, rng.integers(1, 1000, batch),
                                                    rng.integers(1000, 60000, batch)))
        trees = rng.integers(0 if batch > 1 else 1, 65, batch)
        if rng.random() < 0.3:
            trees = np.minimum(trees, rng.integers(1, 4, batch))
        work = int(np.sum(trees * heads * (prefixes + trees)))
        if work <= MAX_WORK and trees.sum() > 0:
            break
        prefixes = prefixes // 2
        if batch > 1 and rng.random() < 0.5:
            batch = max(1, batch // 2)
    total_kv = int(prefixes.sum() + trees.sum())
    num_slots = int(2 ** np.ceil(np.log2(total_kv * 2 + 1024)))
    inst = gen.make_instance(prefixes.tolist(), trees.tolist(), heads, num_slots=num_slots, seed=seed,
                             tree=str(rng.choice(["random", "chain"])), outlier_frac=float(rng.choice([0.0, 0.01])))
    full = bool(rng.random() < 0.3)
    check = full and bool(rng.random() < 0.5)
    contig = bool(rng.random() < 0.3)
    dev_kw = dict(kv_indices_dtype=int(rng.choice([B.I32, B.I64])), out_cache_loc_dtype=int(rng.choice([B.I32, B.I64])),
                  fused_save=bool(rng.random() < 0.25), row_stride=int(rng.choice([576, 576, 640])))
    target = int(rng.choice([0, 0, 0, 5, 64, 256, 700]))
    flags = (B.FLAG_MASK_FULL_ROWS if full else 0) | (B.FLAG_CHECK_PREFIX_MASK if check else 0)
    desc = f"case {case} seed {seed}: B={batch} H={heads} T={int(trees.sum())} Pmax={int(prefixes.max())} full={full} check={check} contig={contig} {dev_kw} target={target}"
    print(desc, flush=True)
    di = DeviceInputs(full_row_instance(inst) if full else inst, **dev_kw)
    tn = int(max(1, trees.max()))
    if contig:
        base = di.num_slots + 16
        extra = torch.full((16 + inst.total_kv + 16, di.pool.shape[1]), -1, dtype=di.pool.dtype, device=di.pool.device)
        di.pool = torch.cat([di.pool, extra]); di.num_slots = di.pool.shape[0]
        vc = Verifier.for_inputs(di, flags=flags, target_items=target, max_tree_nodes=tn)
        out, lse = di.alloc_outputs()
        dst = torch.tensor([base + int(inst.kv_indptr[b]) for b in range(inst.batch)], dtype=torch.int64, device=di.pool.device)
        err = torch.zeros(1, dtype=torch.int32, device=di.pool.device)
        B.compact(vc.plan, vc.args(di, out, lse), dst, err); torch.cuda.synchronize()
        assert int(err.item()) == 0, "compaction error"
        flags |= B.FLAG_CONTIGUOUS_PREFIX
    v = Verifier.for_inputs(di, flags=flags, target_items=target, max_tree_nodes=tn)
    out, lse = di.alloc_outputs()
    out.fill_(float("nan")); lse.fill_(float("nan"))
    v(di, out, lse); torch.cuda.synchronize()
    ew = v.error_word()
    ro, rl, _ = oracle(inst)
    st = gate_stats(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)
    ok = ew == 0 and st["finite"] and st["max_abs"] <= 1e-2 and st["frac_2ulp"] >= 0.999 and st["lse_max_abs"] <= 1e-3 and st["empty_rows_ok"]
    print(f"  err={ew:#x} {st} {'OK' if ok else 'FAIL'}", flush=True)
    if not ok:
        sys.exit(1)
print(f"all {N} cases passed in {time.time() - t_start:.0f} s", flush=True)
