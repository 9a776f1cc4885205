"""Race detection: the readiness protocols under perturbed timing.

A host-set debug knob (tpf_debug_set_delay) makes a seeded subset of the
producer tasks -- GEMM tiles before they bump a chunk's ready counter or an
output tile's counter or store their partials, AllGather copy tasks before
they bump a slice's landed counter -- sleep for a bounded time.  A consumer
that ran before its producer had published (a missing or misplaced wait, a
release or acquire too weak) would then read stale partials or stale
gathered rows.  Every pattern must give exactly the bits of the unfused
baseline run without delays, and every kernel still ends normally (the
sleeps are bounded and far below the waits' own bounds).  The M027 page §04
asks for exactly this check of the ready events."""
import pytest
import torch

from tensor_gemm_reduction_amd import inputs, tpfuse as tp
from tests.parity import assert_bitwise

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def shards(shapes, dist, seed):
    return [inputs.draw(s, dist, seed + i, device=DEV) for i, s in enumerate(shapes)]


# (seed, period, sleeps): 20 patterns, every second to every seventh producer
# sleeping 4 to 40 units (one unit, s_sleep 127, measured about 1 us)
PATTERNS = [(1000 + i, (2, 3, 5, 7)[i % 4], 4 + 9 * ((i * 7) % 5)) for i in range(20)]


def test_reducing_schedulers_under_delays():
    p, M, N, K = 4, 1024, 1024, 256
    X = shards([(M, K)] * p, ("normal", 1.0), 300)
    W = shards([(K, N)] * p, ("normal", 0.05), 310)
    h = tp.Handle(0)
    ref = tp.matmul_allreduce(X, W, torch.float32, n_chunks=1, sched="unfused", handle=h).clone()
    ref_rs = torch.cat(tp.matmul_reducescatter(X, W, torch.bfloat16, n_chunks=1, sched="unfused", handle=h), 0)
    torch.cuda.synchronize()
    for seed, period, sleeps in PATTERNS:
        say(f"delay seed={seed} period={period} sleeps={sleeps}")
        h.set_delay(seed, period, sleeps)
        for sched, n in (("persistent", 4), ("persistent", 8), ("tile", 1), ("two_stream", 4), ("fold", 1)):
            y = tp.matmul_allreduce(X, W, torch.float32, n_chunks=n, sched=sched, handle=h)
            torch.cuda.synchronize()
            assert h.sync_status() == tp.OK, f"{sched}: a bounded wait gave up"
            assert_bitwise(y, ref, f"{sched} n={n} under delay seed={seed} period={period} sleeps={sleeps}")
        ys = torch.cat(tp.matmul_reducescatter(X, W, torch.bfloat16, n_chunks=4, sched="persistent", handle=h), 0)
        torch.cuda.synchronize()
        assert_bitwise(ys, ref_rs, f"reduce-scatter persistent under delay seed={seed}")
    h.set_delay(0, 0, 0)
    h.close()


def test_allgather_under_delays():
    p, Ms, K, N = 8, 64, 512, 768
    Xs = shards([(Ms, K)] * p, ("normal", 1.0), 320)
    W = inputs.draw((K, N), ("normal", 0.05), 330, device=DEV)
    h = tp.Handle(0)
    _, ref = tp.allgather_matmul(Xs, W, torch.bfloat16, n_chunks=1, sched="unfused", handle=h)
    ref = ref.clone()
    torch.cuda.synchronize()
    for seed, period, sleeps in PATTERNS:
        say(f"allgather delay seed={seed} period={period} sleeps={sleeps}")
        h.set_delay(seed, period, sleeps)
        for sched, n in (("persistent", 8), ("persistent", 4), ("two_stream", 8)):
            xg, y = tp.allgather_matmul(Xs, W, torch.bfloat16, n_chunks=n, sched=sched, handle=h)
            torch.cuda.synchronize()
            assert h.sync_status() == tp.OK
            assert torch.equal(xg, torch.cat(Xs, 0)), f"{sched} gathered rows"
            assert_bitwise(y, ref, f"allgather {sched} n={n} under delay seed={seed}")
    h.set_delay(0, 0, 0)
    h.close()


def test_delays_change_timing_not_results():
    """The knob does act: a pattern that delays every task makes the call
    measurably slower (so the patterns above really perturbed the order)."""
    p, M, N, K = 4, 1024, 1024, 256
    X = shards([(M, K)] * p, ("normal", 1.0), 340)
    W = shards([(K, N)] * p, ("normal", 0.05), 350)
    h = tp.Handle(0)

    def timed():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tp.matmul_allreduce(X, W, n_chunks=4, sched="persistent", handle=h)
        torch.cuda.synchronize()
        e0.record()
        tp.matmul_allreduce(X, W, n_chunks=4, sched="persistent", handle=h)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    t_plain = timed()
    h.set_delay(7, 1, 400)        # every task sleeps 400 units (about 0.4 ms)
    t_delay = timed()
    h.set_delay(0, 0, 0)
    assert t_delay > t_plain + 0.1, (t_plain, t_delay)
    h.close()
