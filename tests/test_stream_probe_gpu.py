"""The streaming probe that measures the practical HBM ceiling beside the decode
kernels: it must read every piece of its source once and write the sums the
header promises (integer-valued inputs, so every fp32 sum is exact)."""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_state_read_amd import binding
    binding.lib()


@pytest.mark.timeout(120)
@pytest.mark.parametrize("nt", [False, True], ids=["plain", "streaming"])
@pytest.mark.parametrize("unroll", [4, 8, 16])
@pytest.mark.parametrize("blocks", [0, 3])
def test_probe_writes_exact_sums(unroll, blocks, nt):
    from rank_state_read_amd import binding as B
    chunks = 7
    n4 = chunks * unroll * 256                       # 16-byte pieces read
    src = (torch.arange(4 * n4, device="cuda", dtype=torch.int64) % 1021).to(torch.float32)
    pieces = src.view(chunks, unroll, 256, 4)        # chunk, piece of a thread, thread, lane
    for m in [m for m in (1, 2, 4, 8, 16) if unroll % m == 0]:
        dst = torch.full((n4 // m * 4,), -1.0, device="cuda")
        B.sketchssm_stream_probe(src, 16 * n4, dst, 16 * n4 // m, unroll, blocks, nt)
        torch.cuda.synchronize()
        want = pieces.view(chunks, unroll // m, m, 256, 4).sum(dim=2)
        assert torch.equal(dst.view(chunks, unroll // m, 256, 4), want), m
    if blocks:
        dst = torch.full((blocks * 256 * 4,), -1.0, device="cuda")
        B.sketchssm_stream_probe(src, 16 * n4, dst, 0, unroll, blocks, nt)
        torch.cuda.synchronize()
        # block g sums its chunks g, g + blocks, ... per thread and lane
        want = torch.stack([pieces[g::blocks].sum(dim=(0, 1)) for g in range(blocks)])
        assert torch.equal(dst.view(blocks, 256, 4), want)
