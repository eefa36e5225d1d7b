"""hipGraph capture and replay of the segmented batch.

Eight requests, prefixes U[1000, 185000], trees U[8, 64], H = 8, over a fully
populated 2,097,152-slot pool.  The call is captured once; before each replay
the metadata buffers (qo/kv/mask indptrs, kv_indices, out_cache_loc,
custom_mask) and the queries are rewritten in place, as a serving loop
refreshes its static buffers before replaying ("The Capture-Safe Kernel",
Decision 6).  Every replay must equal an eager call on the same buffers bit
for bit; a few replays are also checked against the oracle on sampled nodes.
"""
import numpy as np
import pytest

from workloads import gen
from tests.gpu_helpers import assert_gate, need_gpu, say

pytestmark = pytest.mark.gpu

N_REPLAYS = 100
ORACLE_REPLAYS = {0, 1, 63, 99}


def _fill(static, rep, torch):
    """Copy one replay's metadata and queries into the static device buffers."""
    def put(name, arr):
        t = torch.from_numpy(np.ascontiguousarray(arr))
        static[name][:t.numel()].copy_(t.reshape(-1).view(static[name].dtype), non_blocking=False)
    put("qo_indptr", rep.qo_indptr)
    put("kv_indptr", rep.kv_indptr)
    put("mask_indptr", rep.mask_indptr)
    put("kv_indices", rep.kv_indices)
    put("out_cache_loc", rep.out_cache_loc)
    put("custom_mask", rep.custom_mask)
    qf = torch.from_numpy(rep.q.view(np.int16))
    static["q"][:qf.shape[0]].copy_(qf)


def test_graph_capture_replay_segmented():
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    from speculative_decoding_mla_page_amd.device import Verifier
    from oracle import mla_verify_ref as R

    bounds = gen.SEGMENTED_BOUNDS
    h = gen.SEGMENTED["num_heads"]
    dev = torch.device("cuda")
    say("segmented: building the 2M-slot pool")
    pool_np = gen.segmented_pool()
    pool = torch.from_numpy(pool_np.view(np.int16)).to(dev)
    mq = bounds["max_q_tokens"]
    static = {
        "q": torch.zeros((mq, h, 576), dtype=torch.int16, device=dev),
        "qo_indptr": torch.zeros(bounds["max_batch"] + 1, dtype=torch.int32, device=dev),
        "kv_indptr": torch.zeros(bounds["max_batch"] + 1, dtype=torch.int32, device=dev),
        "mask_indptr": torch.zeros(bounds["max_batch"] + 1, dtype=torch.int32, device=dev),
        "kv_indices": torch.zeros(bounds["max_kv_tokens"], dtype=torch.int32, device=dev),
        "out_cache_loc": torch.zeros(mq, dtype=torch.int64, device=dev),
        "custom_mask": torch.zeros(mq * bounds["max_tree_nodes"], dtype=torch.uint8, device=dev),
    }
    out_g = torch.zeros((mq, h, 512), dtype=torch.float32, device=dev)
    lse_g = torch.zeros((mq, h), dtype=torch.float32, device=dev)
    out_e = torch.zeros_like(out_g)
    lse_e = torch.zeros_like(lse_g)
    ver = Verifier(h, bounds["max_batch"], mq, bounds["max_kv_tokens"],
                   max_tree_nodes=bounds["max_tree_nodes"])

    def args(out, lse):
        return B.make_args(gen.SEGMENTED["batch"], float(gen.SM_SCALE), static["q"], pool,
                           static["qo_indptr"], static["kv_indptr"], static["kv_indices"],
                           static["out_cache_loc"], static["custom_mask"],
                           static["mask_indptr"], out, lse)

    a_graph = args(out_g, lse_g)
    a_eager = args(out_e, lse_e)

    rep0 = gen.segmented_replay(0)
    _fill(static, rep0, torch)
    torch.cuda.synchronize()
    say("segmented: eager warm-up, then capture")
    B.run(ver.plan, a_eager, ver.workspace)      # loads code objects before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            B.run(ver.plan, a_graph, ver.workspace)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for r in range(N_REPLAYS):
        rep = rep0 if r == 0 else gen.segmented_replay(r)
        _fill(static, rep, torch)
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        og = out_g[:rep.total_q].cpu().numpy()
        lg = lse_g[:rep.total_q].cpu().numpy()
        assert ver.error_word() == 0, f"replay {r}: device error {ver.error_word():#x}"
        # eager call on the same buffers, with a sync in between
        B.run(ver.plan, a_eager, ver.workspace)
        torch.cuda.synchronize()
        oe = out_e[:rep.total_q].cpu().numpy()
        le = lse_e[:rep.total_q].cpu().numpy()
        assert np.array_equal(og, oe) and np.array_equal(lg, le), f"replay {r} != eager"
        if r in ORACLE_REPLAYS:
            rng = np.random.default_rng(r)
            tokens = []
            for b in range(rep.batch):
                q0, t = int(rep.qo_indptr[b]), rep.tree_sizes[b]
                tokens += [q0, q0 + t - 1, q0 + int(rng.integers(0, t))]
            tokens = sorted(set(tokens))
            say(f"segmented replay {r}: oracle on {len(tokens)} nodes, P={rep.prefix_lens}")
            ro, rl, _ = R.mla_verify_reference(rep.q, pool_np, rep.qo_indptr, rep.kv_indptr,
                                               rep.kv_indices, rep.out_cache_loc, rep.custom_mask,
                                               rep.mask_indptr, rep.num_heads, rep.sm_scale,
                                               tokens=tokens)
            assert_gate(og, lg, ro, rl, tokens=tokens, label=f"replay {r}")
        elif r % 20 == 0:
            say(f"segmented replay {r} == eager")
