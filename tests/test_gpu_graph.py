"""GPU: ftmoe_forward captured in a HIP graph.  Every launch of the layer
forward is asynchronous on the caller's stream, allocates nothing and zeroes
what it needs with kernels of that stream, so the whole forward can be
captured once and replayed.  Each replay runs on new token rows written into
the captured input buffer, with eager forwards of the same rows on other
buffers and synchronisations in between; every replay must equal the eager
result bit for bit (ids, weights and output)."""
import numpy as np
import pytest

import block_scaled_fp4_router_amd as ft
import synth
from gpu_util import DEV, layer_pair, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    # layer, T, path, prefill tile layout
    ("c1", 8, "decode", False),
    ("c1-w4a8", 8, "decode", False),
    ("c3", 1, "decode", False),
    ("c0", 16, "prefill", False),
    ("c2", 4096, "prefill", True),
    ("c1-w4a8", 40, "prefill", False),
    ("c4", 64, "prefill", False),
    ("c4-selbias", 8, "decode", False),
    ("c2-bf16", 300, "prefill", False),
]


def _eager(dlay, x, T):
    ws = ft.alloc_workspace(dlay, T)
    y = torch.empty((T, dlay.hidden), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, dlay.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, dlay.top_k), dtype=torch.float32, device=DEV)
    ft.forward(dlay, x, T, ws, y, ids, w)
    torch.cuda.synchronize()
    return y.clone(), ids.clone(), w.clone()


@pytest.mark.parametrize("name,T,path,packed", CASES)
@pytest.mark.timeout(600)
def test_forward_graph_replays_equal_eager(name, T, path, packed):
    say(f"graph capture {name} T={T} path={path} packed={packed}")
    lay, dlay = layer_pair(name, packed=packed)
    dlay = dlay.with_path(path)
    desc = dlay.desc()
    batches = [torch.from_numpy(synth.make_tokens(lay, T, stream=40 + i).view(np.int16)).to(DEV) for i in range(4)]
    x = batches[0].clone()
    ws = ft.alloc_workspace(dlay, T)
    y = torch.empty((T, dlay.hidden), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, dlay.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, dlay.top_k), dtype=torch.float32, device=DEV)
    # one eager call first (per-kernel attributes are set on first use)
    ft.forward(dlay, x, T, ws, y, ids, w, desc=desc)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ft.forward(dlay, x, T, ws, y, ids, w, stream=side, desc=desc)
    torch.cuda.synchronize()
    for i in (1, 2, 3, 0, 2):
        x.copy_(batches[i])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_y, ref_ids, ref_w = _eager(dlay, batches[i], T)
        assert torch.equal(ids, ref_ids), f"replay on batch {i}: ids differ"
        assert torch.equal(w, ref_w), f"replay on batch {i}: weights differ"
        assert torch.equal(y, ref_y), f"replay on batch {i}: output differs"
    say("  5 replays equal the eager forward")
