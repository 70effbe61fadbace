"""moegg_run under HIP graph capture: the library allocates nothing and
clears amax with a kernel (no memset node), so a captured call replays.
Every replay, with eager work and synchronisations between replays, must
reproduce the eager result bit for bit."""
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
