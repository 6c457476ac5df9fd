"""Host-side helpers of bench.py that decide what the summary line reports."""

import bench


def _pieces(N, P, k):
    """Element counts of the instance sub-chunks of a ring AllReduce over P ranks: chunk
    j of P covers [floor(j N / P), floor((j + 1) N / P)), and instance i of k takes the
    same floor partition of that chunk."""
    out = []
    for j in range(P):
        a, b = j * N // P, (j + 1) * N // P
        n = b - a
        out += [(i + 1) * n // k - i * n // k for i in range(k)]
    return out


def test_largest_piece_bound_is_attained_and_never_exceeded():
    for N in (786432, 786432 + 5, 262144, 8 * 24 * 7 + 191, 1000003):
        for P in (4, 8):
            for k in (1, 2, 4, 8, 16, 24, 32):
                assert max(_pieces(N, P, k)) == bench.largest_piece(N, P, k), (N, P, k)


def test_same_launch_treats_slices_covering_the_piece_as_one():
    piece = bench.largest_piece(786432, 8, 24) * 4  # 3 MiB per rank at k = 24: 16 KiB
    assert piece == 16384
    a = (24, 256, 131072, 2, 1)
    assert bench.same_launch(a, (24, 256, 16384, 2, 1), piece)
    assert bench.same_launch(a, (24, 256, 4 << 20, 2, 1), piece)
    assert not bench.same_launch(a, (24, 256, 8192, 2, 1), piece)  # two slices per piece
    assert not bench.same_launch(a, (24, 512, 131072, 2, 1), piece)
    assert not bench.same_launch(a, (32, 256, 131072, 2, 1), piece)
    assert not bench.same_launch(a, (24, 256, 131072, 3, 1), piece)
    assert bench.same_launch((24, 256, 8192, 2, 1), (24, 256, 8192, 2, 1), piece)


def test_ring_factors_follow_the_sweep():
    assert bench.ring_factors(3 << 20) == [1, 2, 4, 8, 16, 24]
    assert bench.ring_factors(32 << 10) == [1, 2, 4, 8, 16, 24]
    assert 32 in bench.ring_factors(32 << 20)
