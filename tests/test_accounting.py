"""The algorithmic work bench.py reports, checked against hand counts."""
import bench


def test_prefill_bytes_long_workload():
    # per token: q, k 2*16*128*2 = 8192; v 48*128*2 = 12288; log_g, beta 8*48 = 384;
    # out 48*128*2 = 12288  -> 33152 B; states: 48 * 128*128*4 * 2 = 6291456 B
    assert bench.prefill_bytes([4576], 16, 48, 128, 128) == 4576 * 33152 + 6291456
    assert bench.prefill_bytes([1168], 16, 48, 128, 128, h0=False) == 1168 * 33152 + 3145728


def test_prefill_flops_one_full_chunk():
    # one chunk of 64 rows, one v-head per k-head, d = 128:
    # 3*64*128*128 + 64*65/2*(128+256) + 64**3/6 + 64*64*128
    mac = 3 * 64 * 128 * 128 + 2080 * 384 + 262144 / 6 + 524288
    assert abs(bench.prefill_flops([64], 1, 1, 128, 128, 64) - 2 * mac) < 1e-6


def test_prefill_flops_long_workload():
    f = bench.prefill_flops([4576], 16, 48, 128, 128, 64)
    assert 28.5e9 < f < 28.6e9   # 71 chunks of 64 + one of 32, 48 v-heads


def test_verify_bytes():
    b = bench.verify_bytes(16, 16, 48, 128, 128)
    assert b == 16 * 48 * 65536 + 16 * 4 * (2 * 16 * 128 + 48 * 128) * 2 + 16 * 4 * 48 * 8 \
        + 16 * 4 * 48 * 128 * 2 + 16 * 48 * (4 * 128 * 4 + 16 + 4 * 128 * 2)
    assert 54e6 < b < 55e6


def test_fold_bytes():
    # two sequences folded (na = 1 and 4), one not (na = 0)
    assert bench.fold_bytes([0, 1, 4], 48, 128, 128) == 48 * (131072 + 1 * 768 + 16) + 48 * (131072 + 4 * 768 + 16)  # state 64 KiB read + write


def test_step_bytes():
    # 16 sequences x 48 v-heads: state 64 KiB read + write; one row of q, k (2 x 16 x 128 bf16),
    # v (48 x 128 bf16), gate and beta (48 x 8 B); out (48 x 128 bf16)
    b = bench.step_bytes(16, 16, 48, 128, 128)
    assert b == 16 * 48 * 131072 + 16 * (8192 + 12288) + 16 * 384 + 16 * 12288
    assert 101e6 < b < 101.3e6
