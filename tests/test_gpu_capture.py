"""hipGraph capture and replay of the segmented batch.

Eight requests, prefixes U[1000, 185000], trees U[8, 64], H = 8, over a fully
populated 2,097,152-slot pool.  The call is captured once; before each replay
the metadata buffers (qo/kv/mask indptrs, kv_indices, out_cache_loc,
custom_mask) and the queries are rewritten in place, as a serving loop
refreshes its static buffers before replaying ("The Capture-Safe Kernel",
Decision 6).  Every replay must equal an eager call on the same buffers bit
for bit and leave every output row finite; every tenth replay (and the last)
is compared with the oracle on all of its nodes.  out, lse and the workspace
sit between guard bands of a fixed bit pattern that must survive all replays
(a write past either end of any of them would change it).

The same capture runs a second time with the contiguous-prefix fast path:
before each replay every request's prefix indices are rewritten as one
contiguous run from a random base (the pool is fully populated), as a
compacted pool would hold them.
"""
import copy
import functools

import numpy as np
import pytest

from workloads import gen
from tests.gpu_helpers import assert_gate, assert_rows_finite, need_gpu, say

pytestmark = pytest.mark.gpu

N_REPLAYS = 100
ORACLE_REPLAYS = set(range(0, N_REPLAYS, 10)) | {N_REPLAYS - 1}
N_REPLAYS_CONTIG = 20
GUARD_BYTES = 64 * 1024          # each side; a multiple of 256 keeps the workspace aligned
CANARY = 0x5AC3E11D              # guard word (a NaN-free float bit pattern)


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


@functools.lru_cache(maxsize=1)
def _pool_np():
    return gen.segmented_pool()


def _contiguous(rep, r, num_slots):
    """The replay with each request's prefix indices one run from a random base."""
    rng = np.random.default_rng(9000 + r)
    out = copy.copy(rep)
    kvi = np.asarray(rep.kv_indices).copy()
    kvp = np.asarray(rep.kv_indptr)
    for b in range(len(kvp) - 1):
        n = int(kvp[b + 1] - kvp[b])
        if n:
            base = int(rng.integers(0, num_slots - n))
            kvi[kvp[b]:kvp[b + 1]] = base + np.arange(n)
    out.kv_indices = kvi.astype(np.asarray(rep.kv_indices).dtype)
    return out


class Guarded:
    """A device buffer of `nbytes` between two guard bands of CANARY words."""

    def __init__(self, torch, nbytes, device):
        self.g = GUARD_BYTES // 4
        self.n = (nbytes + 3) // 4
        self.store = torch.full((self.g * 2 + self.n,), CANARY, dtype=torch.int32, device=device)
        self.torch = torch

    def body(self, dtype, shape=None):
        t = self.store[self.g:self.g + self.n].view(dtype)
        return t if shape is None else t[:int(np.prod(shape))].view(shape)

    def intact(self) -> bool:
        lo = self.store[:self.g]
        hi = self.store[self.g + self.n:]
        return bool((lo == CANARY).all().item()) and bool((hi == CANARY).all().item())


@pytest.mark.parametrize("contig", [False, True], ids=["index_path", "contiguous_prefix"])
def test_graph_capture_replay_segmented(contig):
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    from oracle import mla_verify_ref as R
    n_replays = N_REPLAYS_CONTIG if contig else N_REPLAYS
    oracle_replays = ({0, n_replays // 2, n_replays - 1} if contig else ORACLE_REPLAYS)

    bounds = gen.SEGMENTED_BOUNDS
    h = gen.SEGMENTED["num_heads"]
    dev = torch.device("cuda")
    say("segmented: building the 2M-slot pool")
    pool_np = _pool_np()
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
    cfg = B.make_config(h, bounds["max_batch"], mq, bounds["max_kv_tokens"],
                        max_tree_nodes=bounds["max_tree_nodes"],
                        flags=B.FLAG_CONTIGUOUS_PREFIX if contig else 0)
    plan = B.plan(cfg)
    ws_bytes = B.workspace_size(plan)
    g_out = Guarded(torch, mq * h * 512 * 4, dev)
    g_lse = Guarded(torch, mq * h * 4, dev)
    g_ws = Guarded(torch, ws_bytes, dev)
    out_g = g_out.body(torch.float32, (mq, h, 512))
    lse_g = g_lse.body(torch.float32, (mq, h))
    ws = g_ws.body(torch.uint8)[:ws_bytes]
    assert ws.data_ptr() % 256 == 0
    out_e = torch.zeros_like(out_g)
    lse_e = torch.zeros_like(lse_g)
    ws_e = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def args(out, lse):
        return B.make_args(gen.SEGMENTED["batch"], float(gen.SM_SCALE), static["q"], pool,
                           static["qo_indptr"], static["kv_indptr"], static["kv_indices"],
                           static["out_cache_loc"], static["custom_mask"],
                           static["mask_indptr"], out, lse)

    def error_word(w):
        return int(w[:4].view(torch.int32).item()) & 0xFFFFFFFF

    a_graph = args(out_g, lse_g)
    a_eager = args(out_e, lse_e)

    def replay(r):
        rep = gen.segmented_replay(r)
        return _contiguous(rep, r, pool_np.shape[0]) if contig else rep

    rep0 = replay(0)
    _fill(static, rep0, torch)
    torch.cuda.synchronize()
    say("segmented: eager warm-up, then capture")
    B.run(plan, a_eager, ws_e)      # loads code objects before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            B.run(plan, a_graph, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert g_out.intact() and g_lse.intact() and g_ws.intact(), "capture wrote outside its buffers"

    for r in range(n_replays):
        rep = rep0 if r == 0 else replay(r)
        _fill(static, rep, torch)
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        og = out_g[:rep.total_q].cpu().numpy()
        lg = lse_g[:rep.total_q].cpu().numpy()
        assert error_word(ws) == 0, f"replay {r}: device error {error_word(ws):#x}"
        assert_rows_finite(og, lg, label=f"replay {r}")
        # eager call on the same buffers, with a sync in between
        B.run(plan, a_eager, ws_e)
        torch.cuda.synchronize()
        oe = out_e[:rep.total_q].cpu().numpy()
        le = lse_e[:rep.total_q].cpu().numpy()
        assert np.array_equal(og, oe) and np.array_equal(lg, le), f"replay {r} != eager"
        if r in oracle_replays:
            say(f"segmented replay {r}: oracle on all {rep.total_q} nodes, P={rep.prefix_lens} "
                f"T={rep.tree_sizes}")
            ro, rl, _ = R.mla_verify_reference(rep.q, pool_np, rep.qo_indptr, rep.kv_indptr,
                                               rep.kv_indices, rep.out_cache_loc, rep.custom_mask,
                                               rep.mask_indptr, rep.num_heads, rep.sm_scale)
            assert_gate(og, lg, ro, rl, label=f"segmented replay {r}")
            assert g_out.intact() and g_lse.intact() and g_ws.intact(), f"guard band hit by replay {r}"
    assert g_out.intact() and g_lse.intact() and g_ws.intact(), "guard band hit"
