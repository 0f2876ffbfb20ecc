"""The library's calls inside a captured HIP graph.

Each call launches kernels only: it allocates nothing, never synchronises and
never reads device memory on the host, so a serving loop can capture it once
and replay it.  Each test captures one step on a side stream, replays it
several times with eager work and host synchronisations between the replays,
and requires every replay to reproduce the eager result bit for bit (the
kernels are deterministic: fixed work split, fixed reduction order)."""
import numpy as np
import pytest
import torch

from workloads import gen

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


def _capture(step):
    """Capture step() on a side stream (after one eager warm-up call there)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    return g


def _replays_match(gu, g, outs, ref, disturb):
    for i in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan")) if t.is_floating_point() else t.fill_(-1)
        disturb()                     # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            got = t.detach().cpu()
            assert torch.equal(got.view(torch.uint8), r.view(torch.uint8)), f"replay {i} differs from the eager run"


def test_decode_in_a_graph(gu):
    case = gen.make_decode_case(name="graph_decode", seed=95, B=8, Hq=16, Hk=4, D=128, q_dtype="bf16",
                                kv_dtype="e4m3fn", seq_lens=[1, 64, 65, 300, 1000, 2047, 5, 129])
    gu.announce("graph decode")
    dd = gu.DeviceDecode(case)
    dd.run()
    torch.cuda.synchronize()
    ref = [dd.out.detach().cpu().clone(), dd.lse.detach().cpu().clone()]
    g = _capture(dd.run)
    scratch = torch.randn(1 << 20, device="cuda")
    _replays_match(gu, g, [dd.out, dd.lse], ref, lambda: scratch.mul_(1.0001))


def test_prefill_bf16_and_fp8_in_a_graph(gu):
    cases = [gen.make_prefill_case(name="graph_mla", seed=96, seq_lens=[130, 64, 1, 400], Hq=8, Hk=8, D_qk=192,
                                   D_rope=64, D_v=128),
             gen.make_prefill_fp8_case(name="graph_fp8", seed=97, seq_lens=[130, 64, 1, 400], Hq=8, Hk=2, D_rope=64,
                                       blockwise=True)]
    for case in cases:
        gu.announce(f"graph prefill {case.name}")
        dp = gu.DevicePrefill(case)
        dp.run()
        torch.cuda.synchronize()
        ref = [dp.out.detach().cpu().clone(), dp.lse.detach().cpu().clone()]
        g = _capture(dp.run)
        scratch = torch.randn(1 << 20, device="cuda")
        _replays_match(gu, g, [dp.out, dp.lse], ref, lambda: scratch.add_(1.0))


@pytest.mark.parametrize("kv_dtype", ["bf16", "e4m3fn"])
def test_chunk_step_in_a_graph(gu, kv_dtype):
    """A chunked-prefill step (append, then attention) captured together, over
    a bf16 and over an fp8 cache.  The append writes the same bytes on every
    replay, so the cache and the output must match the eager step exactly."""
    case = gen.make_chunk_case(name="graph_chunk", seed=98, prefix_lens=[100, 0, 640], q_lens=[28, 64, 129], Hq=8,
                               Hk=2, D_rope=64, kv_dtype=kv_dtype)
    gu.announce(f"graph chunk step, {kv_dtype} cache")
    dc = gu.DeviceChunk(case)

    def step():
        dc.append()
        dc.run()

    step()
    torch.cuda.synchronize()
    ref = [dc.out.detach().cpu().clone(), dc.lse.detach().cpu().clone(), dc.k_pool.detach().cpu().clone()]
    g = _capture(step)
    scratch = torch.randn(1 << 20, device="cuda")
    _replays_match(gu, g, [dc.out, dc.lse], ref[:2], lambda: scratch.mul_(0.999))
    assert torch.equal(dc.k_pool.detach().cpu().view(torch.uint8), ref[2].view(torch.uint8))


@pytest.mark.parametrize("kv_dtype", ["bf16", "e4m3fn"])
def test_short_chunk_step_in_a_graph(gu, kv_dtype):
    """A multi-token decode step (append of 1..4 tokens per sequence, then
    the attention on the decode workers) captured together; every replay
    reproduces the eager step bit for bit."""
    case = gen.make_chunk_case(name="graph_short", seed=99, prefix_lens=[100, 0, 640, 63, 2000],
                               q_lens=[4, 1, 3, 4, 2], Hq=16, Hk=4, kv_dtype=kv_dtype)
    gu.announce(f"graph short-chunk step, {kv_dtype} cache")
    dc = gu.DeviceChunk(case)
    assert dc.plan.kernel == (6 if kv_dtype == "e4m3fn" else 5)

    def step():
        dc.append()
        dc.run()

    step()
    torch.cuda.synchronize()
    ref = [dc.out.detach().cpu().clone(), dc.lse.detach().cpu().clone()]
    g = _capture(step)
    scratch = torch.randn(1 << 20, device="cuda")
    _replays_match(gu, g, [dc.out, dc.lse], ref, lambda: scratch.mul_(0.999))
