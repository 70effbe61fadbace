"""moegg_run under HIP graph capture and on concurrent streams.

The library allocates nothing, keeps no state between calls and clears amax
with a kernel (no memset node), so a captured call replays and calls on
different streams do not interfere.  Every graph replay, with eager work and
synchronisations between replays, must reproduce the eager result bit for
bit, and so must each of two problems run concurrently on two streams."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mg = pytest.importorskip("moe_grouped_block_amd")
from moe_grouped_block_amd import plumbing as pl  # noqa: E402

CASES = {
    # FP8 D / D_col with row and column scales
    "graph_swiglu_fp8": ("fc1_swiglu_l8", dict(L=3, K=512, N=320, routing=("topk", 300, 2))),
    # bf16 D with the per-group amax the library clears itself
    "graph_gating_bf16_amax": ("quant_gating_l4", dict(L=4, K=256, N=288, routing=("multinomial", 400))),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name):
    base, over = CASES[name]
    case = synth.make_case(base, seed=3100 + sorted(CASES).index(name), name=name, **over)
    p = case.problem
    print(f"\n[gpu-case] {name} graph capture valid_m={p['valid_m']} n={p['n']} k={p['k']}", flush=True)
    dev = pl.to_device(case.arrays)
    inputs = pl.inputs_for(p, dev)

    eager = pl.empty_outputs(p, fill=0xA5)
    mg.run(p, {**inputs, **eager})
    torch.cuda.synchronize()
    ref = pl.to_host(eager)

    outs = pl.empty_outputs(p, fill=0xA5)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # warm-up off the default stream
        mg.run(p, {**inputs, **outs})
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mg.run(p, {**inputs, **outs})
    torch.cuda.synchronize()

    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for rep in range(4):
        for t in outs.values():                # stale contents the replay must overwrite
            t.view(torch.uint8).fill_(0x5A + rep)
        junk.uniform_()                        # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = pl.to_host(outs)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), f"replay {rep}: {k} differs from the eager call"
    del graph


def test_concurrent_streams_match_serial():
    """Two different problems enqueued on two streams at once (the library
    keeps no state between calls): each result equals its serial run."""
    cases = [synth.make_case("fc1_swiglu_l8", seed=3201, name="streams_a", L=3, K=512, N=320,
                             routing=("topk", 300, 2)),
             synth.make_case("srelu_tanh_fp4_l32", seed=3202, name="streams_b", L=3, K=512, N=256,
                             routing=("multinomial", 300))]
    for c in cases:
        print(f"\n[gpu-case] {c.name} two streams valid_m={c.problem['valid_m']}", flush=True)
    devs = [pl.to_device(c.arrays) for c in cases]
    serial = []
    for c, d in zip(cases, devs):
        o = pl.empty_outputs(c.problem, fill=0xA5)
        mg.run(c.problem, {**pl.inputs_for(c.problem, d), **o})
        torch.cuda.synchronize()
        serial.append(pl.to_host(o))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [pl.empty_outputs(c.problem, fill=0x5A) for c in cases]
    torch.cuda.synchronize()
    for _ in range(3):
        for c, d, o, s in zip(cases, devs, outs, streams):
            mg.run(c.problem, {**pl.inputs_for(c.problem, d), **o}, stream=s)
    torch.cuda.synchronize()
    for c, o, ref in zip(cases, outs, serial):
        got = pl.to_host(o)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), f"{c.name}: {k} differs from the serial run"
