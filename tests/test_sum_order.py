"""How often does the association order of the binary64 sum of squares change the
binary32 1/RMS?  The oracle adds the squares sequentially in h; the row kernel adds
each lane's 8*VPT squares in order, then combines lanes with a fixed butterfly
(xor 1, xor 2, the other quad, the other 8, the other 16, then lanes 0 + 32) and
waves in order.  This test replays both orders in float64 on 20000 random BF16
rows (W=4 H=2048 layout: 256 lanes x 1 vector, 4 waves) and counts rows whose
rounded 1/RMS differ.  It documents why norm_out is held to "within 2 BF16 steps"
rather than bit-identity, and that in practice the two agree (expected count 0;
the probability per row is about 2^-29)."""
import numpy as np

from tests.bf16util import bf16_values


def kernel_order_sum(sq):
    """sq: [rows, 2048] float64 squares; lane l owns elements 8l..8l+7 (one vector)."""
    rows = sq.shape[0]
    lane = np.zeros((rows, 256))
    for e in range(8):                      # per-lane sequential accumulation from 0
        lane = lane + sq.reshape(rows, 256, 8)[:, :, e]
    waves = lane.reshape(rows, 4, 64)

    def partner(v, idx):
        return v[:, :, idx]
    i = np.arange(64)
    x = waves
    x = x + partner(x, i ^ 1)
    x = x + partner(x, i ^ 2)
    x = x + partner(x, (i & ~7) | (7 - (i & 7)))      # row_half_mirror
    x = x + partner(x, (i & ~15) | (15 - (i & 15)))   # row_mirror
    x = x + partner(x, i ^ 16)
    wave_sum = x[:, :, 0] + x[:, :, 32]
    total = wave_sum[:, 0]
    for w in range(1, 4):
        total = total + wave_sum[:, w]
    return total


def test_sum_order_rarely_changes_inverse_rms():
    rng = np.random.default_rng(12345)
    rows, H = 20000, 2048
    eps = np.float32(1e-6)
    diffs = 0
    for chunk in range(4):
        vals = rng.standard_normal((rows // 4, H)) * np.sqrt(5.0)
        bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # truncation is fine here
        ro = bf16_values(bits)
        sq = ro * ro
        seq = np.zeros(rows // 4)
        for h in range(H):                  # the oracle's order
            seq = seq + sq[:, h]
        tree = kernel_order_sum(sq)
        inv_seq = (1.0 / np.sqrt(seq / H + float(eps))).astype(np.float32)
        inv_tree = (1.0 / np.sqrt(tree / H + float(eps))).astype(np.float32)
        diffs += int((inv_seq != inv_tree).sum())
        assert np.allclose(seq, tree, rtol=1e-13)
    assert diffs <= 1, diffs
