"""The MFMA-loop measurement helper that gives the achievable dense bf16 rate:
its per-thread sums are exact and linear in the round count, and their total
matches a closed form of the operands the kernel builds."""
import numpy as np
import pytest

from tests.gpu_helpers import need_gpu, say

pytestmark = pytest.mark.gpu


def _expected_total(blocks: int, iters: int) -> float:
    # lane l supplies row/column l % 16 and k-group l // 16 (eight k each) of
    # the 16x32 A and 32x16 B operands, with A = (l + j) / 1024 and
    # B = (l - j) / 1024 for its j-th k; the sum of all entries of A.B only
    # depends on which lanes share a k, not on the order of k inside a group
    a = np.zeros((16, 32))
    b = np.zeros((32, 16))
    for lane in range(64):
        for j in range(8):
            a[lane % 16, 8 * (lane // 16) + j] = (lane + j) / 1024
            b[8 * (lane // 16) + j, lane % 16] = (lane - j) / 1024
    per_chain = float((a @ b).sum())
    return per_chain * 4 * 4 * blocks * iters      # 4 chains, 4 waves per workgroup


def test_mfma_loop_is_exact_and_linear():
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    blocks = 12
    say(f"calibrate_mfma blocks={blocks} iters=1,3")
    out1 = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    out3 = torch.full_like(out1, float("nan"))
    B.calibrate_mfma(1, blocks, out1)
    B.calibrate_mfma(3, blocks, out3)
    torch.cuda.synchronize()
    o1 = out1.cpu().numpy().astype(np.float64)
    o3 = out3.cpu().numpy().astype(np.float64)
    assert np.isfinite(o1).all() and np.isfinite(o3).all()
    assert np.array_equal(o3, 3 * o1)
    assert o1.sum() == _expected_total(blocks, 1)


def test_mfma_loop_rejects_small_output():
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    out = torch.empty(255, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        B.calibrate_mfma(1, 1, out)


def test_read_stream_reads_every_unit_once():
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    # a size that leaves a partial last stride, and words whose checksum is known
    blocks = 3
    units = blocks * 256 * 5 + 77
    gen = np.random.default_rng(5)
    words = gen.integers(0, 1 << 20, size=(units, 4), dtype=np.uint32)
    say(f"calibrate_read blocks={blocks} units={units}")
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    B.calibrate_read(buf, blocks, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # thread t reads units t, t + stride, ...; its sum of (w0 ^ w1) + (w2 ^ w3)
    # stays below 2^24, so the float it writes is exact
    per_unit = (words[:, 0] ^ words[:, 1]).astype(np.int64) + (words[:, 2] ^ words[:, 3])
    stride = blocks * 256
    want = np.zeros(stride, dtype=np.int64)
    np.add.at(want, np.arange(units) % stride, per_unit)
    assert want.max() < (1 << 24)
    assert np.array_equal(got.astype(np.int64), want)
