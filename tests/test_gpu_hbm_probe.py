"""The streaming probe (safe_hbm_probe) does what its header says: the read form returns, per
thread, the xor of the 32-bit words of the 16-byte chunks that thread owns (chunk c belongs to
thread c mod the thread count), recomputed here with numpy; the copy form copies every byte;
bad arguments are refused before launch."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")


def expected_words(words: np.ndarray, threads: int) -> np.ndarray:
    chunk = np.bitwise_xor.reduce(words.reshape(-1, 4), axis=1)
    pad = (-chunk.size) % threads
    chunk = np.concatenate([chunk, np.zeros(pad, np.uint32)])
    return np.bitwise_xor.reduce(chunk.reshape(-1, threads), axis=0)


@pytest.mark.parametrize("nchunks,blocks", [(1, 1), (255, 1), (5000, 3), (3 * 4 * 768 + 17, 3), (1 << 16, 16)])
def test_read_words_and_copy(nchunks, blocks):
    g = torch.Generator(device="cpu").manual_seed(nchunks)
    src_h = torch.randint(-(1 << 31), (1 << 31) - 1, (nchunks * 4,), generator=g, dtype=torch.int64).to(torch.int32)
    src = src_h.cuda()
    got = sq.hbm_probe(src, blocks)
    torch.cuda.synchronize()
    want = expected_words(src_h.numpy().view(np.uint32), blocks * 256)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want)
    dst = torch.full_like(src, 7)
    sq.hbm_probe(src, blocks, dst=dst)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), src_h)


def test_bad_arguments_are_refused():
    buf = torch.zeros(1024, dtype=torch.int32, device="cuda")
    out = torch.zeros(256, dtype=torch.int32, device="cuda")
    lib = sq.lib
    p, o = buf.data_ptr(), out.data_ptr()
    assert lib.safe_hbm_probe(2, p, None, 4096, 1, o, None) == -4          # mode
    assert lib.safe_hbm_probe(0, p, None, 0, 1, o, None) == -2             # bytes
    assert lib.safe_hbm_probe(0, p, None, 4100, 1, o, None) == -2          # not a multiple of 16
    assert lib.safe_hbm_probe(0, p, None, 4096, 0, o, None) == -4          # blocks
    assert lib.safe_hbm_probe(0, p, None, 4096, 1, None, None) == -1       # read without out
    assert lib.safe_hbm_probe(1, p, None, 2048, 1, None, None) == -1       # copy without dst
    assert lib.safe_hbm_probe(0, p + 4, None, 1024, 1, o, None) == -8      # misaligned
    assert lib.safe_hbm_probe(1, p, p + 16, 2048, 1, None, None) == -4     # overlapping copy
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0 and torch.count_nonzero(buf).item() == 0
