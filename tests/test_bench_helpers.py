"""Host-side helpers of bench.py that decide what the summary line reports."""

import bench


def test_instance_pieces_tile_each_chunk_on_the_16_byte_grid():
    """Pieces cover each program chunk exactly, in order; every offset from the chunk's
    start but its length is a multiple of the alignment, so equal-length chunks get equal
    pieces; no piece exceeds ceil(len / k) + align - 1."""
    for N in (786432, 786432 + 5, 262144, 8 * 24 * 7 + 191, 1000003, 33554424):
        for P in (4, 8, 24):
            for k in (1, 2, 4, 8, 16, 24, 32):
                for align in (4, 8):
                    for j in range(P):
                        lo, hi = j * N // P, (j + 1) * N // P
                        b = bench.instance_bounds(lo, hi, k, align)
                        assert b[0] == lo and b[-1] == hi and len(b) == k + 1
                        assert all(b[i] <= b[i + 1] for i in range(k))
                        assert all((x - lo) % align == 0 for x in b[:-1])
                        assert [x - lo for x in b] == [x for x in bench.instance_bounds(0, hi - lo, k, align)]
                        assert max(b[i + 1] - b[i] for i in range(k)) <= -(-(hi - lo) // k) + align - 1


def test_largest_piece_of_the_headline():
    assert bench.largest_piece(786432, 8, 24) == 4096   # 3 MiB per rank: 98,304-element chunks / 24
    assert bench.largest_piece(262144, 8, 24) == 1368   # 1 MiB: 1365.3 elements, bounds on the 4-element grid
    assert bench.largest_piece(786432, 8, 32) == 3072


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
    assert {32, 48, 64} <= set(bench.ring_factors(32 << 20))


def test_committed_traffic_records_describe_tunable_launches():
    """The headline's traffic record is taken at a launch the headline's tuner can pick
    (a factor of the 3 MiB sweep's set); every record's traffic is its fetch plus write
    bytes (each rounded to a byte), within 5 % of its plan bytes (no wasted re-reads at these sizes)."""
    import json
    import os
    for mib, factors in ((3, bench.CONFIG_FACTORS), (32, bench.ring_factors(32 << 20)),
                         (256, bench.ring_factors(256 << 20))):
        path = os.path.join(bench.ROOT, "profiles", f"executor_ring_ar_8r_{mib}mib_traffic.json")
        with open(path) as fh:
            t = json.load(fh)
        k, nt, sl, proto, kern = t["config"]
        assert k in factors and nt in bench.TUNE_THREADS and sl in bench.TUNE_SLICES
        assert proto in bench.PROTOCOLS and kern == bench.KERNEL
        assert abs(t["bytes_per_launch"] - t["fetch_bytes_per_launch"] - t["write_bytes_per_launch"]) <= 1  # rounding
        assert abs(t["bytes_per_launch"] / t["plan_bytes_per_launch"] - 1) < 0.05
        assert len(t["source_digest"]) == 16
