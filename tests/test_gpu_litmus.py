"""Message-passing litmus test of the executor's transfer-store policy (release /
acquire across workgroups on the same and on different XCDs), through the C ABI.

Each round a producer workgroup writes fresh words with plain stores and sets a flag
(plain store when the consumer runs on its XCD, agent-scope release otherwise); the
consumer polls the flag and reads the words with agent-coherent loads, exactly as the
executor's receives do. Any stale word would be counted; every wait is bounded."""

import pytest

from chunk_schedule_execution_amd import capi

pytestmark = pytest.mark.gpu


def case(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("cross", [False, True])
@pytest.mark.parametrize("words", [3072, 65536])
def test_message_passing_sees_every_round(cross, words):
    import torch
    rounds = 2000 if words <= 4096 else 200
    case(f"litmus message passing cross_xcd={cross} words={words} rounds={rounds}")
    res = capi.ccl_litmus_message_passing(cross, rounds, words, 200000, torch.cuda.current_stream().cuda_stream)
    for p, (pxcd, cxcd, done, bad, first_round, first_word, plain_flags, expired) in enumerate(res):
        assert expired == 0, (p, res[p])
        assert bad == 0 and first_round == 0, (p, res[p])
        assert done == rounds, (p, res[p])
        if cross:
            assert pxcd != cxcd and plain_flags == 0, (p, res[p])  # every flag is a full release
        elif pxcd == cxcd:
            assert plain_flags == rounds, (p, res[p])  # the plain-store path was the one tested
    if not cross:  # workgroup ids congruent mod 8 land on one XCD under the round-robin dispatch
        assert sum(1 for r in res if r[0] == r[1]) >= 6, res


@pytest.mark.parametrize("ll", [False, True])
@pytest.mark.parametrize("two_operands", [False, True])
@pytest.mark.parametrize("hops,nbytes,nthreads,window", [(15, 16384, 256, 0), (15, 16384, 256, 4 << 20),
                                                         (4, 1 << 20, 1024, 0), (31, 16, 64, 0), (3, 48, 128, 4096)])
def test_hop_probe_chain_delivers_every_launch(ll, two_operands, hops, nbytes, nthreads, window):
    """The hop-latency probe runs the executor's slice code (or, with ll, its low-latency
    protocol) along a chain of workgroups:
    every launch's new source arrives unchanged at the end of the chain (adding the zero
    operand keeps the bits), also where launches step through a window (a payload off
    the 256-byte grid of the window's steps included), no wait expires, and each
    hand-off takes a positive time
    below the watchdog's. (Placement is reported, not asserted: a chain workgroup on
    another XCD gets a full release, as in the executor.)"""
    import torch
    launches = 10
    case(f"hop probe hops={hops} bytes={nbytes} two_operands={two_operands} nthreads={nthreads} window={window} ll={ll}")
    us, (off_xcd, expired, wrong, done) = capi.ccl_hop_probe(
        hops, nbytes, two_operands, nthreads, launches, window_bytes=window, timeout_us=200000,
        stream=torch.cuda.current_stream().cuda_stream, ll=ll)
    print(f"[hop] {sorted(us)[launches // 2]:.3f} us per hand-off, {off_xcd} chain workgroups off XCD 0", flush=True)
    assert expired == 0 and wrong == 0 and done == launches, (off_xcd, expired, wrong, done)
    assert len(us) == launches and all(0 < u < 1000 for u in us), us
