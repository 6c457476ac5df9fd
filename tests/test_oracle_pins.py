"""Pins of the CPU oracle against what the definitions and arithmetic fix.

Nothing here re-types an oracle formula to compare it with itself: every check is a
hand-worked fixture (tests/golden), a closed form, a library routine (torch's bf16
cast and add), a brute-force search, an error bound, or an identity between two
different oracle functions (composition, degenerate group shapes).
"""

import numpy as np
import pytest
import torch

from oracle import definitions as O1
from oracle import numerics as nm
from oracle import program as prog
from oracle import schedule_order as O2
import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def ints(row):
    return [int(v) for v in row]


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rne_golden(golden):
    for fp32_hex, bf16_hex, *_ in golden("bf16_rne_cases.txt"):
        x = np.array([int(fp32_hex, 16)], dtype=np.uint32).view(np.float32)
        assert int(nm.f32_to_bf16_rne(x)[0]) == int(bf16_hex, 16), fp32_hex


def test_bf16_widen_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0x8000], dtype=np.uint16)
    got = nm.bf16_to_f32(bits).astype(np.float64)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 2.0**-133
    assert np.isinf(got[3]) and got[4] == 0.0 and np.signbit(got[4])


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # add dense clusters of ties and near-ties
    ties = (rng.integers(0, 2**16, size=20_000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    bits = np.concatenate([bits, ties, ties + 1, ties - 1])
    f = bits.view(np.float32)
    ours = nm.f32_to_bf16_rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN in -> NaN out, same sign
    o = nm.bf16_to_f32(ours[nan])
    assert np.all(np.isnan(o))
    assert np.array_equal(np.signbit(o), np.signbit(f[nan]))


def _nearest_bf16_bruteforce(v64):
    """Nearest bf16 to each float64 value by trying neighbours; ties to even bits."""
    out = np.empty(len(v64), dtype=np.uint16)
    for i, v in enumerate(v64):
        f32 = np.float32(v)
        k = int(np.array([f32], np.float32).view(np.uint32)[0] >> 16)
        best = None
        for cand in (k - 1, k, k + 1, k + 2):
            cand &= 0xFFFF
            cv = float(nm.bf16_to_f32(np.array([cand], np.uint16))[0])
            if np.isnan(cv):
                continue
            if np.isinf(cv):
                cv = np.copysign(2.0**128, cv)  # rounding treats inf as the next binade
            d = abs(cv - v)
            key = (d, cand & 1)
            if np.signbit(cv) != np.signbit(v) and v != 0:
                continue
            if best is None or key < best[0]:
                best = (key, cand)
        out[i] = best[1]
    return out


def test_bf16_rne_matches_bruteforce_nearest():
    rng = np.random.default_rng(11)
    f = np.concatenate([rng.standard_normal(3000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e30).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32)])
    got = nm.f32_to_bf16_rne(f)
    want = _nearest_bf16_bruteforce(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_add_is_correctly_rounded_and_matches_torch():
    # Two bf16 operands: the fp32 sum is exact or rounded once with 24 >= 2*8+2 bits,
    # so rounding it to bf16 equals rounding the exact sum (double rounding is
    # innocuous). Check against the brute-force nearest of the exact float64 sum,
    # and against torch's own bf16 addition.
    rng = np.random.default_rng(5)
    a = W.normal_bf16_bits(4000, rng)
    b = W.normal_bf16_bits(4000, rng)
    b[:500] = nm.f32_to_bf16_rne(nm.bf16_to_f32(b[:500]) * np.float32(2.0**-12))  # wide exponent gaps
    got = nm.add_stored(a, b, "bf16")
    exact = nm.bf16_to_f32(a).astype(np.float64) + nm.bf16_to_f32(b).astype(np.float64)
    assert np.array_equal(got, _nearest_bf16_bruteforce(exact))
    ta = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)
    tref = (ta + tb).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, tref)


def test_i32_wraps():
    a = np.array([2**31 - 1, -(2**31), 5], dtype=np.int32)
    b = np.array([1, -1, -7], dtype=np.int32)
    assert nm.add_stored(a, b, "i32").tolist() == [-(2**31), 2**31 - 1, -2]


def test_f32_add_is_correctly_rounded():
    rng = np.random.default_rng(3)
    a = rng.standard_normal(10000).astype(np.float32)
    b = (rng.standard_normal(10000) * 1e-6).astype(np.float32)
    got = nm.add_stored(a, b, "f32")
    want = (a.astype(np.float64) + b.astype(np.float64)).astype(np.float32)  # exact sum, one rounding
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- O1 definitions

def _brute_allreduce(xs):
    n = len(xs[0])
    return [sum(float(x[i]) for x in xs) for i in range(n)]


@pytest.mark.parametrize("P", [1, 2, 3, 4])
@pytest.mark.parametrize("N", [1, 5, 12])
def test_o1_allreduce_bruteforce(P, N):
    xs = W.make_inputs("normal_f32", N, P, cfg_id=99)
    ref = O1.allreduce(xs, "f32")
    assert np.allclose(ref.exact, _brute_allreduce(xs), rtol=0, atol=1e-12)
    assert np.allclose(ref.abs_sum, [sum(abs(float(x[i])) for x in xs) for i in range(N)])


def test_o1_allreduce_p1_is_identity_and_int_exact():
    x = W.make_inputs("int_f32", 100, 1, cfg_id=99)
    assert np.array_equal(O1.allreduce(x, "f32").exact, x[0].astype(np.float64))
    xi = [np.array([2**31 - 1, 3], np.int32), np.array([1, -5], np.int32)]
    assert O1.allreduce(xi, "i32").exact.tolist() == [-(2**31), -2]


def test_o1_copy_collectives_golden(golden):
    rows = golden("copy_collectives_provenance.txt")
    i = 0
    while i < len(rows):
        name, _, P, _, N = rows[i]
        P, N = int(P), int(N)
        ys = [ints(r[1:]) for r in rows[i + 1:i + 1 + P]]
        xs = [W.provenance_i32(N, r) for r in range(P)]
        if name == "alltoall":
            got = O1.alltoall(xs)
        elif name == "allgather":
            got = [O1.allgather(xs) for _ in range(P)]
        else:
            got = O1.alltonext(xs, [np.full(N, -1, np.int32)] * P)
        for r in range(P):
            assert np.asarray(got[r]).tolist() == ys[r], (name, r)
        i += 1 + P


@pytest.mark.parametrize("P,b", [(2, 3), (4, 5), (8, 16), (32, 7)])
def test_o1_alltoall_provenance_decode(P, b):
    xs = [W.provenance_i32(P * b, r) for r in range(P)]
    ys = O1.alltoall(xs)
    for r in range(P):
        y = ys[r].astype(np.int64)
        src, idx = y >> 20, y & (2**20 - 1)
        pos = np.arange(P * b)
        assert np.array_equal(src, pos // b)              # block s came from rank s
        assert np.array_equal(idx, r * b + pos % b)       # ... from its block r


def test_o1_reducescatter_golden(golden):
    rows = {r[0]: ints(r[1:]) for r in golden("reducescatter_p2.txt")}
    xs = [np.array(rows["x0"], np.int32), np.array(rows["x1"], np.int32)]
    got = O1.reducescatter(xs, "i32")
    assert got[0].exact.tolist() == rows["y0"] and got[1].exact.tolist() == rows["y1"]


def test_o1_grouped_forms_compose_to_allreduce():
    G, L, N = 3, 4, 24
    xs = W.make_inputs("int_f32", N, G * L, cfg_id=98)
    rs = O1.reducescatter_intra(xs, "f32", L)
    ar = O1.allreduce_inter([s.exact for s in rs], "f32", L)
    ag = O1.allgather_intra([a.exact for a in ar], L)
    full = O1.allreduce(xs, "f32").exact
    for r in range(G * L):
        assert np.array_equal(ag[r], full)


# ---------------------------------------------------------------- O2 ring

def _fixture(golden, name):
    rows = golden(name)
    d = {r[0]: r[1:] for r in rows}
    return d


@pytest.mark.parametrize("name", ["ring_allreduce_p4_order.txt", "ring_allreduce_p3_blocks.txt"])
def test_o2_ring_allreduce_golden(golden, name):
    d = _fixture(golden, name)
    P, C = int(d["P"][0]), int(d["nchunks"][0])
    xs = [np.array(ints(d[f"x{r}"]), np.float32) for r in range(P)]
    ys = O2.ring_allreduce(xs, C, "f32")
    for y in ys:
        assert y.astype(np.int64).tolist() == ints(d["y"])


def test_o2_ring_p2_is_correctly_rounded_sum():
    xs = W.make_inputs("normal_f32", 4099, 2, cfg_id=97)
    ys = O2.ring_allreduce(xs, 2, "f32")
    want = (xs[0].astype(np.float64) + xs[1].astype(np.float64)).astype(np.float32)
    assert all(np.array_equal(y, want) for y in ys)


def test_o2_ring_p1_is_copy():
    xs = W.make_inputs("normal_f32", 33, 1, cfg_id=97)
    assert np.array_equal(O2.ring_allreduce(xs, 3, "f32")[0], xs[0])


@pytest.mark.parametrize("P,C,N", [(2, 2, 7), (3, 3, 10), (3, 6, 64), (4, 4, 63), (4, 8, 5), (8, 8, 1000)])
def test_o2_ring_integer_inputs_exact(P, C, N):
    xs = W.make_inputs("int_f32", N, P, cfg_id=96)
    exact = O1.allreduce(xs, "f32").exact
    for y in O2.ring_allreduce(xs, C, "f32"):
        assert np.array_equal(y.astype(np.float64), exact)


@pytest.mark.parametrize("P", [3, 4, 8, 16])
def test_o2_ring_within_summation_bound(P):
    xs = W.make_inputs("normal_f32", 5000, P, cfg_id=95)
    ref = O1.allreduce(xs, "f32")
    ys = O2.ring_allreduce(xs, P, "f32")
    # recursive summation of P terms: |err| <= (P-1) u sum|x| + O(u^2), u = 2^-24
    bound = (P - 1) * 2.0**-24 * (1 + 1e-6)
    assert nm.scaled_error(ys[0], ref.exact, ref.abs_sum, "f32") <= bound
    assert all(np.array_equal(ys[0], y) for y in ys)


def test_o2_ring_reducescatter_is_allreduce_shard():
    P, C, N = 4, 8, 120
    xs = W.make_inputs("normal_f32", N, P, cfg_id=94)
    ar = O2.ring_allreduce(xs, C, "f32")[0]
    rs = O2.ring_reducescatter(xs, C, "f32")
    n = N // P
    for r in range(P):
        assert np.array_equal(rs[r], ar[r * n:(r + 1) * n])


def test_o2_bf16_ring_within_bound():
    P, N = 8, 4000
    xs = W.make_inputs("normal_bf16", N, P, cfg_id=93)
    ref = O1.allreduce(xs, "bf16")
    y = O2.ring_allreduce(xs, P, "bf16")[0]
    # every stored partial is rounded to bf16 (u = 2^-8): error <= (P-1) u sum|x| (+ u^2 terms)
    assert nm.scaled_error(y, ref.exact, ref.abs_sum, "bf16") <= (P - 1) * 2.0**-8 * 1.01


# ---------------------------------------------------------------- O2 hierarchical / 2-D

def test_o2_hier_golden(golden):
    d = _fixture(golden, "hier_allreduce_g2l2.txt")
    G, L = int(d["G"][0]), int(d["L"][0])
    xs = [np.array(ints(d[f"x{r}"]), np.float32) for r in range(G * L)]
    for y in O2.hierarchical_allreduce(xs, G, L, "f32"):
        assert y.astype(np.int64).tolist() == ints(d["y"])


@pytest.mark.parametrize("L", [2, 3, 5, 8])
def test_o2_hier_g1_is_ring_over_l(L):
    xs = W.make_inputs("normal_f32", 333, L, cfg_id=92)
    assert np.array_equal(O2.hierarchical_allreduce(xs, 1, L, "f32")[0], O2.ring_allreduce(xs, L, "f32")[0])


@pytest.mark.parametrize("G", [2, 3, 4])
def test_o2_hier_l1_is_ring_over_g(G):
    xs = W.make_inputs("normal_f32", 100, G, cfg_id=92)
    assert np.array_equal(O2.hierarchical_allreduce(xs, G, 1, "f32")[0], O2.ring_allreduce(xs, G, "f32")[0])


@pytest.mark.parametrize("dtype,kind", [("f32", "normal_f32"), ("bf16", "normal_bf16")])
def test_o2_hier_equals_three_stage_composition(dtype, kind):
    G, L, N = 2, 4, 8 * 37
    xs = W.make_inputs(kind, N, G * L, cfg_id=91)
    fused = O2.hierarchical_allreduce(xs, G, L, dtype)
    s1 = O2.ring_reducescatter_intra(xs, L, dtype)
    s2 = O2.ring_allreduce_inter(s1, L, dtype)
    s3 = O1.allgather_intra(s2, L)
    for r in range(G * L):
        assert np.array_equal(s3[r], fused[r])


def test_o2_hier_integer_exact_and_bf16_bound():
    G, L, N = 2, 8, 1024
    xs = W.make_inputs("int_f32", N, G * L, cfg_id=90)
    exact = O1.allreduce(xs, "f32").exact
    for y in O2.hierarchical_allreduce(xs, G, L, "f32"):
        assert np.array_equal(y.astype(np.float64), exact)
    xb = W.make_inputs("normal_bf16", N, G * L, cfg_id=90)
    ref = O1.allreduce(xb, "bf16")
    yb = O2.hierarchical_allreduce(xb, G, L, "bf16")
    assert all(np.array_equal(yb[0], y) for y in yb)
    # depth of the association tree is (L-1) + (G-1) roundings
    assert nm.scaled_error(yb[0], ref.exact, ref.abs_sum, "bf16") <= (L + G - 2) * 2.0**-8 * 1.01


@pytest.mark.parametrize("L", [2, 3, 4])
def test_o2_rs2d_degenerate_shapes_are_ring(L):
    xs = W.make_inputs("normal_f32", 12 * L, L, cfg_id=89)
    ring = O2.ring_reducescatter(xs, L, "f32")
    a = O2.reducescatter_2d(xs, 1, L, "f32")
    b = O2.reducescatter_2d(xs, L, 1, "f32")
    for r in range(L):
        assert np.array_equal(a[r], ring[r]) and np.array_equal(b[r], ring[r])


def test_o2_rs2d_integer_exact():
    G, L, N = 3, 8, 24 * 11
    xs = W.make_inputs("int_f32", N, G * L, cfg_id=88)
    ref = O1.reducescatter(xs, "f32")
    got = O2.reducescatter_2d(xs, G, L, "f32")
    for r in range(G * L):
        assert np.array_equal(got[r].astype(np.float64), ref[r].exact)


def _rs2d_on_golden(golden, name, fn):
    d = _fixture(golden, name)
    G, L = int(d["G"][0]), int(d["L"][0])
    xs = [np.array(ints(d[f"x{r}"]), np.float32) for r in range(G * L)]
    got = fn(xs, G, L, "f32")
    return [int(np.asarray(y).astype(np.int64)[0]) for y in got], d


@pytest.mark.parametrize("name", ["reducescatter_2d_g2l2_order.txt", "reducescatter_2d_g2l3_chain.txt"])
def test_o2_rs2d_golden(golden, name):
    """Hand-worked fixtures fix the 2-D ReduceScatter's association: inside the group
    first (chain from lane l+1 to the owning lane l), then across the groups."""
    got, d = _rs2d_on_golden(golden, name, O2.reducescatter_2d)
    assert got == ints(d["y"])


def _rs2d_variant(xs, G, L, dtype, cross_first=False, owner_first=False, wrong_map=False):
    """Plausible slips in a 2-D ReduceScatter, for the planted-mistake test below."""
    n = len(xs[0]) // (G * L)
    out = []
    for b in range(G * L):
        l, h = divmod(b, G) if wrong_map else (b % L, b // L)
        lo, hi = b * n, (b + 1) * n
        lane_order = [(l + t) % L for t in range(L)] if owner_first else [(l + 1 + t) % L for t in range(L)]
        group_order = [(h + 1 + t) % G for t in range(G)]
        if cross_first:
            parts = [O2.fold([np.asarray(xs[g * L + ln][lo:hi]) for g in group_order], dtype) for ln in lane_order]
        else:
            parts = [O2.fold([np.asarray(xs[g * L + ln][lo:hi]) for ln in lane_order], dtype) for g in group_order]
        out.append(O2.fold(parts, dtype))
    return out


def test_rs2d_variant_harness_is_the_oracle_when_unplanted(golden):
    for name in ("reducescatter_2d_g2l2_order.txt", "reducescatter_2d_g2l3_chain.txt"):
        got, d = _rs2d_on_golden(golden, name, _rs2d_variant)
        assert got == ints(d["y"])


# ---------------------------------------------------------------- program interpreter

# A 2-rank AllReduce written out by hand: rank 1 sends its chunk 0 to rank 0, which
# adds its own; rank 0 sends its chunk 1 to rank 1 likewise; then the results are
# copied back. (MSCCLang report, section 3.1: copy/reduce on chunks of
# input/output/scratch buffers.)
AR2 = [
    ("copy", 1, "in", 0, 0, "out", 0, 1), ("reduce", 0, "in", 0, 0, "out", 0, 1),
    ("copy", 0, "in", 1, 1, "out", 1, 1), ("reduce", 1, "in", 1, 1, "out", 1, 1),
    ("copy", 0, "out", 0, 1, "out", 0, 1), ("copy", 1, "out", 1, 0, "out", 1, 1),
]


def test_program_interpreter_two_rank_allreduce():
    xs = W.make_inputs("normal_f32", 77, 2, cfg_id=87)
    ys = prog.run_program(AR2, xs, "f32", 2, 2, 0)
    want = (xs[0].astype(np.float64) + xs[1].astype(np.float64)).astype(np.float32)
    assert np.array_equal(ys[0], want) and np.array_equal(ys[1], want)
    assert prog.check_postcondition(AR2, "allreduce", 2, 2, 0)


def test_program_interpreter_ring_p3_by_hand_matches_golden(golden):
    # The 3-rank ring of the golden fixture (two chunks per rank), written out op
    # by op: chunk j (owner o = j // 2) goes o+1 -> o+2 (partial in scratch) -> o
    # (into out), then out is forwarded o -> o+1 -> o+2.
    ops = []
    for j in range(6):
        o = j // 2
        a, b = (o + 1) % 3, (o + 2) % 3
        ops += [("copy", a, "in", j, b, "scr", j, 1), ("reduce", b, "in", j, b, "scr", j, 1),
                ("copy", b, "scr", j, o, "out", j, 1), ("reduce", o, "in", j, o, "out", j, 1),
                ("copy", o, "out", j, a, "out", j, 1), ("copy", a, "out", j, b, "out", j, 1)]
    d = _fixture(golden, "ring_allreduce_p3_blocks.txt")
    xs = [np.array(ints(d[f"x{r}"]), np.float32) for r in range(3)]
    ys = prog.run_program(ops, xs, "f32", 6, 6, 6)
    for y in ys:
        assert y.astype(np.int64).tolist() == ints(d["y"])
    assert prog.check_postcondition(ops, "allreduce", 3, 6, 6)


def test_symbolic_rejects_a_ring_that_skips_a_rank():
    bad = [op for op in AR2 if op != ("reduce", 0, "in", 0, 0, "out", 0, 1)]
    with pytest.raises(AssertionError):
        prog.check_postcondition(bad, "allreduce", 2, 2, 0)
    dup = AR2 + [("reduce", 0, "in", 0, 0, "out", 0, 1)]
    with pytest.raises(AssertionError):
        prog.check_postcondition(dup, "allreduce", 2, 2, 0)


def test_program_interpreter_rejects_length_mismatch_and_input_writes():
    xs = W.make_inputs("normal_f32", 10, 2, cfg_id=86)
    with pytest.raises(ValueError):  # chunk 0 has 3 elements, chunk 1 has 4 (N=7, C=2)
        prog.run_program([("copy", 0, "in", 0, 1, "out", 1, 1)], [x[:7] for x in xs], "f32", 2, 2, 0)
    with pytest.raises(ValueError):
        prog.run_symbolic([("copy", 0, "in", 0, 1, "in", 0, 1)], 2, 2, 2, 0)


# ---------------------------------------------------------------- error metric

def test_scaled_error_cases():
    exact = np.array([1.0, 0.0, -3.0])
    abs_sum = np.array([3.0, 0.0, 3.0])
    assert nm.scaled_error(np.array([1.0, 0.0, -3.0], np.float32), exact, abs_sum, "f32") == 0.0
    assert nm.scaled_error(np.array([1.5, 0.0, -3.0], np.float32), exact, abs_sum, "f32") == 0.5 / 3
    assert nm.scaled_error(np.array([1.0, 1e-30, -3.0], np.float32), exact, abs_sum, "f32") == float("inf")


def test_elementwise_rel_error_cases():
    """Hand-worked: only elements whose exact sum is at least 1e-3 of their magnitude
    sum count; all-zero columns never do."""
    exact = np.array([1.0, 0.0, -3.0, 1e-4])
    abs_sum = np.array([3.0, 0.0, 3.0, 2.0])
    y = np.array([1.5, 0.0, -2.7, 5.0], np.float32)
    # kept: elements 0 (|1| >= 0.003) and 2 (|-3| >= 0.003); element 3 (1e-4 < 0.002) is not
    assert nm.elementwise_rel_error(y, exact, abs_sum, "f32") == pytest.approx(0.5)
    y2 = np.array([1.0, 0.0, -2.7, 5.0], np.float32)
    assert nm.elementwise_rel_error(y2, exact, abs_sum, "f32") == pytest.approx(0.3 / 3.0, rel=1e-6)
    assert nm.elementwise_rel_error(y2, exact, abs_sum, "f32", floor=1e-5) == pytest.approx((5.0 - 1e-4) / 1e-4, rel=1e-6)
    assert nm.elementwise_rel_error(np.zeros(2, np.float32), np.zeros(2), np.zeros(2), "f32") == 0.0


@pytest.mark.parametrize("P", [4, 8, 24])
def test_elementwise_rel_error_within_derived_bound(P):
    """Recursive summation: |y - s| <= (P-1) u sum|x| (u = 2^-24, up to O(u^2)); on the
    kept elements |s| >= 1e-3 sum|x|, so the plain relative error is at most
    (P-1) u 1e3 there. The chain-order oracle stays inside it; adding one input twice
    (a planted duplicate addend) does not."""
    xs = W.make_inputs("normal_f32", 20000, P, cfg_id=84)
    ref = O1.allreduce(xs, "f32")
    y = O2.ring_allreduce(xs, P, "f32")[0]
    bound = (P - 1) * 2.0**-24 * 1e3 * (1 + 1e-6)
    assert nm.elementwise_rel_error(y, ref.exact, ref.abs_sum, "f32") <= bound
    bad = O2.add_stored(y, xs[0], "f32")
    assert nm.elementwise_rel_error(bad, ref.exact, ref.abs_sum, "f32") > bound


# ---------------------------------------------------------------- O2 tree

def _golden_tree_ok(golden):
    d = _fixture(golden, "tree_allreduce_p3_order.txt")
    P, C = int(d["P"][0]), int(d["nchunks"][0])
    xs = [np.array(ints(d[f"x{r}"]), np.float32) for r in range(P)]
    return O2.tree_allreduce(xs, C, "f32")[0].astype(np.int64).tolist() == ints(d["y"])


def test_o2_tree_allreduce_golden(golden):
    """Hand-worked association of the tree: (child 2t+2 + root) + child 2t+1, which
    rounds differently from the ring's chain on these inputs."""
    assert _golden_tree_ok(golden)
    d = _fixture(golden, "tree_allreduce_p3_order.txt")
    xs = [np.array(ints(d[f"x{r}"]), np.float32) for r in range(3)]
    assert O2.ring_allreduce(xs, 3, "f32")[0].astype(np.int64).tolist() == ints(d["ring"])


def test_o2_tree_small_cases():
    xs = W.make_inputs("normal_f32", 4099, 2, cfg_id=97)
    want = (xs[0].astype(np.float64) + xs[1].astype(np.float64)).astype(np.float32)
    assert all(np.array_equal(y, want) for y in O2.tree_allreduce(xs, 2, "f32"))
    xs = W.make_inputs("normal_f32", 33, 1, cfg_id=97)
    assert np.array_equal(O2.tree_allreduce(xs, 3, "f32")[0], xs[0])
    for P, C, N in ((3, 6, 64), (5, 5, 99), (8, 16, 1000)):
        xs = W.make_inputs("int_f32", N, P, cfg_id=96)
        exact = O1.allreduce(xs, "f32").exact
        for y in O2.tree_allreduce(xs, C, "f32"):
            assert np.array_equal(y.astype(np.float64), exact)


@pytest.mark.parametrize("P,c,dtype", [(3, 1, "f32"), (5, 2, "f32"), (8, 1, "bf16"), (8, 2, "f32"), (6, 1, "bf16")])
def test_tree_program_follows_the_documented_association(P, c, dtype):
    """The sequential interpreter of the tree program (the DSL's semantics) lands on
    exactly the documented tree order, in both storage types."""
    from chunk_schedule_execution_amd import programs
    pr = programs.tree_allreduce(P, c)
    kind = "normal_bf16" if dtype == "bf16" else "normal_f32"
    xs = W.make_inputs(kind, 301, P, cfg_id=94)
    got = prog.run_program(pr.as_tuples(), xs, dtype, pr.in_chunks, pr.out_chunks, pr.scratch_chunks)
    want = O2.tree_allreduce(xs, pr.in_chunks, dtype)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


# ---------------------------------------------------------------- the pins bite

def _golden_ring_ok(golden, name):
    d = _fixture(golden, name)
    P, C = int(d["P"][0]), int(d["nchunks"][0])
    xs = [np.array(ints(d[f"x{r}"]), np.float32) for r in range(P)]
    return O2.ring_allreduce(xs, C, "f32")[0].astype(np.int64).tolist() == ints(d["y"])


def test_planted_mistakes_fail_the_pins(golden, monkeypatch):
    """Plausible slips in the oracle (reversed ring, chain starting at the owner,
    round-robin ownership, a dropped bf16 rounding) each fail a pin above."""
    def reversed_ring(xs, lo, hi, owner, dtype):
        P = len(xs)
        order = [(owner - 1 - t) % P for t in range(P)]
        return O2.fold([np.asarray(xs[r][lo:hi]) for r in order], dtype)

    def owner_first(xs, lo, hi, owner, dtype):
        P = len(xs)
        order = [(owner + t) % P for t in range(P)]
        return O2.fold([np.asarray(xs[r][lo:hi]) for r in order], dtype)

    for bad in (reversed_ring, owner_first):
        with monkeypatch.context() as m:
            m.setattr(O2, "_ring_chunk", bad)
            assert not _golden_ring_ok(golden, "ring_allreduce_p4_order.txt")

    def tree_children_swapped(xs, lo, hi, owner, dtype):  # (child 2t+1 + root) + child 2t+2
        P = len(xs)

        def partial(t):
            x = np.asarray(xs[(owner + t) % P][lo:hi])
            kids = [u for u in (2 * t + 1, 2 * t + 2) if u < P]
            if not kids:
                return x.copy()
            acc = nm.add_stored(partial(kids[0]), x, dtype)
            for u in kids[1:]:
                acc = nm.add_stored(acc, partial(u), dtype)
            return acc
        return partial(0)

    def tree_as_chain(xs, lo, hi, owner, dtype):  # the root added last
        P = len(xs)
        return O2.fold([np.asarray(xs[(owner + t) % P][lo:hi]) for t in range(1, P)] + [xs[owner][lo:hi]], dtype)

    for bad in (tree_children_swapped, tree_as_chain):
        with monkeypatch.context() as m:
            m.setattr(O2, "_tree_chunk", bad)
            assert not _golden_tree_ok(golden)
            if bad is tree_children_swapped:  # and lands where the fixture works it out by hand
                d = _fixture(golden, "tree_allreduce_p3_order.txt")
                xs = [np.array(ints(d[f"x{r}"]), np.float32) for r in range(3)]
                assert O2.tree_allreduce(xs, 3, "f32")[0].astype(np.int64).tolist() == ints(d["swapped"])

    real = O2._ring_chunk
    with monkeypatch.context() as m:
        # own chunk j by j mod P instead of by block
        m.setattr(O2, "_ring_chunk", lambda xs, lo, hi, owner, dtype: real(xs, lo, hi, lo % len(xs), dtype))
        assert not _golden_ring_ok(golden, "ring_allreduce_p3_blocks.txt")

    # the 2-D ReduceScatter: stages swapped, chain starting at the owning lane, blocks
    # mapped to (group, lane) the wrong way round; each fails a fixture and lands where
    # the fixture works it out by hand
    for kw, row, name in ((dict(cross_first=True), "swapped", "reducescatter_2d_g2l2_order.txt"),
                          (dict(owner_first=True), "owner_first", "reducescatter_2d_g2l3_chain.txt"),
                          (dict(wrong_map=True), "wrong_map", "reducescatter_2d_g2l3_chain.txt")):
        with monkeypatch.context() as m:
            m.setattr(O2, "reducescatter_2d", lambda xs, G, L, dtype, kw=kw: _rs2d_variant(xs, G, L, dtype, **kw))
            got, d = _rs2d_on_golden(golden, name, O2.reducescatter_2d)
            assert got != ints(d["y"]) and got == ints(d[row]), kw

    with monkeypatch.context() as m:
        m.setattr(nm, "f32_to_bf16_rne", lambda x: (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16))
        cases = golden("bf16_rne_cases.txt")
        x = np.array([int(c[0], 16) for c in cases], dtype=np.uint32).view(np.float32)
        assert [int(v) for v in nm.f32_to_bf16_rne(x)] != [int(c[1], 16) for c in cases]


def test_sampled_folds_match_whole_folds():
    P, N = 8, 1003
    xs = W.make_inputs("normal_f32", N, P, cfg_id=85)
    full = O2.ring_allreduce(xs, 16, "f32")[0]
    idx = np.arange(N)
    assert np.array_equal(O2.ring_allreduce_at(xs, 16, idx, "f32"), full)
    xb = W.make_inputs("normal_bf16", 16 * 37, 16, cfg_id=85)
    fullh = O2.hierarchical_allreduce(xb, 2, 8, "bf16")[0]
    assert np.array_equal(O2.hierarchical_allreduce_at(xb, 2, 8, np.arange(16 * 37), "bf16"), fullh)
