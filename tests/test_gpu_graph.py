"""Decode steps captured in a HIP graph (as a serving loop would run them) give the same results
as the same steps issued eagerly: the decode entry point launches one kernel per call and no
memset or allocation, so it can be captured. The graph is replayed several times, with eager
work (restoring the caches) and synchronisation between replays, and every replay is compared
bit for bit with the eager run."""
from __future__ import annotations

import pytest

import workloads
from gpu_util import gpu_decode, gpu_prefill, make_case, say, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_depthwise_amd as axon

    axon.load()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_decode_graph_replays_match_eager(act):
    B, E, L, steps = 4, 1000, 20, 6
    say(f"[graph] decode B={B} E={E} act={act}, {steps} captured steps")
    inp, extra = make_case(B, L, E, act, seed=70, caches=True)
    d = to_device(inp)
    _, cache0, state0 = gpu_prefill(d, conv_cache_in=torch.from_numpy(extra["conv_cache_in"]).cuda(),
                                    ssm_state_in=torch.from_numpy(extra["ssm_state_in"]).cuda())
    w = workloads.Workload(0, "graph", "decode", B, L, E, act)
    adt = torch.bfloat16 if act == "bf16" else torch.float32
    ins = []
    for s in range(steps):
        st = workloads.decode_step_inputs(w, s)
        ins.append({k: torch.from_numpy(st[k]).cuda().to(adt) for k in st})

    # eager
    cache, state = cache0.clone(), state0.clone()
    ys_ref = [gpu_decode(ins[s], d, cache, state).clone() for s in range(steps)]
    torch.cuda.synchronize()
    cache_ref, state_ref = cache.clone(), state.clone()

    # captured: static cache / state / outputs
    cache_g, state_g = cache0.clone(), state0.clone()
    ys_g = [torch.empty_like(ys_ref[0]) for _ in range(steps)]
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for s in range(steps):
                gpu_decode(ins[s], d, cache_g, state_g, y=ys_g[s], stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        cache_g.copy_(cache0)
        state_g.copy_(state0)
        for y in ys_g:
            y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(ys_g[s], ys_ref[s]), f"replay {rep}, step {s}: y differs"
        assert torch.equal(cache_g, cache_ref), f"replay {rep}: conv cache differs"
        assert torch.equal(state_g, state_ref), f"replay {rep}: state differs"
