"""The matrix-core rate probe (safe_mfma_probe) computes what its header says: for each wave,
the sum of its lanes' checksums equals the sum of every product of the 16 MFMAs it issued,
recomputed here in float64 from the documented operand draw (32-bit mixer, bf16 rounding)
and operand layouts -- so the probe's rate counts real products on the stated operands."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")

M32 = 0xFFFFFFFF


def mix(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.uint64) & M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def bf16_rne(v: np.ndarray) -> np.ndarray:
    b = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def fragments(seed: int, lanes: np.ndarray) -> np.ndarray:
    """[lanes, 16 fragments, 8 elements] operand values (A: fragments 0-7, B: 8-15)."""
    f = np.arange(16)[None, :, None]
    e = np.arange(8)[None, None, :]
    c = lanes[:, None, None].astype(np.uint64) * 64 + (f * 8 + e).astype(np.uint64)
    h = mix(np.uint64(seed) ^ mix(c)) >> 8
    return bf16_rne((h.astype(np.float64) / 16777216.0 - 0.5) * 4.0)


@pytest.mark.parametrize("shape", [32, 16])
def test_probe_sums_are_the_products_it_claims(shape):
    blocks, seed = 3, 12345
    got = sq.mfma_probe(shape, 1, blocks, seed=seed).cpu().numpy().astype(np.float64)
    lanes = np.arange(blocks * 256)
    v = fragments(seed, lanes)
    group = 32 if shape == 32 else 16          # lanes sharing a k range: lane // group
    for w in range(blocks * 4):
        fr = v[64 * w:64 * (w + 1)]            # [64, 16, 8]
        h = np.arange(64) // group
        # column sums of A / row sums of B per (k range, element): the sum over all outputs of
        # one MFMA is sum_k (sum_i A[i, k]) (sum_j B[k, j])
        sums = np.stack([fr[h == g].sum(axis=0) for g in range(64 // group)])   # [groups, 16, 8]
        expect = 0.0
        for q in range(16):
            fa, fb = q % 8, 8 + (q + q // 8) % 8
            expect += float((sums[:, fa, :] * sums[:, fb, :]).sum())
        total = float(got[64 * w:64 * (w + 1)].sum())
        mag = float(np.abs(fr).sum()) * 8.0
        assert abs(total - expect) <= 1e-5 * mag + 1e-3, (shape, w, total, expect)


def test_probe_rejects_bad_arguments():
    for args in ((8, 1, 1), (32, 0, 1), (16, 1, 0), (32, 1 << 25, 1)):
        with pytest.raises(sq.SafeError) as e:
            sq.mfma_probe(*args)
        assert e.value.status == -4
