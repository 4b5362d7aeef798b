"""GPU: the allocation-free forward (ftmoe_forward_noalloc, the library's own
fixed scratch instead of a caller workspace) against ftmoe_forward on the
same inputs: the same kernels on the same bytes, so routing, weights and
outputs must be equal bit for bit, and the outputs within the parity bar of
the oracle.  Two calls in a row, the second on a smaller batch (the scratch
keeps the first call's contents), per layer; decode and a small prefill."""
import numpy as np
import pytest

import block_scaled_fp4_router_amd as ft
import oracle
import synth
from gpu_util import DEV, bf16_dev_to_f64, layer_pair, rel_fro, run_forward, say, to_dev_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def noalloc_forward(dlay, x_bits):
    T = x_bits.shape[0]
    x = to_dev_bf16(x_bits)
    y = torch.empty((T, dlay.hidden), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, dlay.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, dlay.top_k), dtype=torch.float32, device=DEV)
    ft.forward_noalloc(dlay, x, T, y, ids, w)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(y), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("name,T1,T2", [("c1", 8, 3), ("c3", 16, 1), ("c1-w4a8", 8, 5), ("c0", 300, 70),
                                        ("c0", 16, 5)])
@pytest.mark.timeout(300)
def test_noalloc_forward_equals_forward(name, T1, T2):
    lay, dlay = layer_pair(name)
    for T in (T1, T2):
        say(f"noalloc forward {name} T={T}")
        x = synth.make_tokens(lay, T, stream=50 + T)
        y, ids, w = noalloc_forward(dlay, x)
        ry, rids, rw = run_forward(dlay, x)
        assert np.array_equal(ids, rids) and np.array_equal(w, rw)
        assert np.array_equal(y, ry), "allocation-free forward differs from ftmoe_forward"
        ref = oracle.forward(lay, x)
        assert np.array_equal(ids, ref["ids"])
        err = rel_fro(y, ref["y"])
        say(f"  rel_fro vs oracle {err:.3e}")
        assert err <= (3e-2 if lay.cfg.act in ("fp8", "mxfp8") else 2e-2)


@pytest.mark.timeout(300)
def test_noalloc_forward_refuses_a_batch_beyond_its_scratch():
    lay, dlay = layer_pair("c2")
    T = 4096
    assert ft.workspace_size(dlay, T) > 32 << 20
    x = torch.zeros((T, dlay.hidden), dtype=torch.int16, device=DEV)
    y = torch.full((T, dlay.hidden), 77, dtype=torch.int16, device=DEV)
    with pytest.raises(ft.FtmoeError) as e:
        ft.forward_noalloc(dlay, x, T, y)
    assert e.value.status == ft.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 77).all())   # nothing enqueued
