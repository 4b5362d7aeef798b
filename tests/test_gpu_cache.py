"""GPU: the expert-slot pool (ftmoe_cache_*).  The routed experts live in
pinned host memory and are copied into a device pool of a few slots as the
steps need them; the outputs must equal ftmoe_forward's on the same layer
with its experts in device memory bit for bit (the same kernels run on the
same bytes), whether a step fits the slots (one pass: hits and misses) or
not (several passes), in the decode and prefill paths.  The counters must
match the step's distinct experts."""
import numpy as np
import pytest

import block_scaled_fp4_router_amd as ft
import synth
from gpu_util import DEV, bf16_dev_to_f64, layer_pair, run_forward, say, to_dev_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _small(name, H, E, k, I, fmt, act="bf16", Is=0):
    cfg = synth.LayerConfig(name, (16,), H, E, k, I, fmt, act=act, shared_inter=Is, seed=9)
    return synth.make_layer(cfg, cache=False)


def cache_forward(cache, x_bits):
    T = x_bits.shape[0]
    x = to_dev_bf16(x_bits)
    ws = cache.workspace(T)
    y = torch.empty((T, cache.layer.hidden), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, cache.layer.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, cache.layer.top_k), dtype=torch.float32, device=DEV)
    cache.forward(x, T, ws, y, ids, w)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(y), ids.cpu().numpy(), w.cpu().numpy()


CASES = [
    # name, layer, T, path, slots
    ("c1", None, 8, "decode", 64),
    ("c1", None, 8, "decode", 12),
    ("c1-w4a8", None, 8, "decode", 20),
    ("c1", None, 40, "prefill", 24),
    ("nvs", (256, 16, 4, 128, "nvfp4", "bf16", 128), 9, "decode", 5),
    ("nvs", (256, 16, 4, 128, "nvfp4", "bf16", 128), 70, "prefill", 5),
    ("f8a8", (256, 8, 2, 256, "fp8", "fp8", 0), 12, "decode", 8),
    ("f8a8", (256, 8, 2, 256, "fp8", "fp8", 0), 300, "prefill", 8),
    ("bf16", (256, 8, 2, 256, "bf16", "bf16", 0), 70, "prefill", 3),
]


@pytest.mark.parametrize("name,shape,T,path,slots", CASES)
@pytest.mark.timeout(600)
def test_cache_forward_equals_device_layer(name, shape, T, path, slots):
    say(f"expert cache {name} T={T} path={path} slots={slots}")
    if shape is None:
        lay, dlay = layer_pair(name)
    else:
        lay = _small(name, *shape)
        dlay = ft.DeviceLayer.from_host(lay, DEV)
    x = synth.make_tokens(lay, T, stream=T)
    ref_y, ref_ids, ref_w = run_forward(dlay, x, path)
    cache = ft.ExpertCache.from_host(lay, slots, DEV, path=path)
    y, ids, w = cache_forward(cache, x)
    assert np.array_equal(ids, ref_ids) and np.array_equal(w, ref_w)
    assert np.array_equal(y, ref_y)
    n = len(np.unique(ids))
    st = cache.stats()
    passes = -(-n // slots)
    say(f"  distinct experts {n}, stats {st}")
    assert st["passes"] == passes
    assert st["hits"] + st["misses"] == n
    assert st["misses"] == n   # a fresh pool
    per_expert = sum(t.numel() * t.element_size() for t in (cache.host_gate_up.codes, cache.host_gate_up.block_scales,
                                                           cache.host_gate_up.tensor_scales, cache.host_down.codes,
                                                           cache.host_down.block_scales,
                                                           cache.host_down.tensor_scales) if t is not None) // dlay.num_experts
    assert st["bytes_copied"] == n * per_expert
    # the same step again: everything that stayed resident is a hit
    y2, ids2, _ = cache_forward(cache, x)
    assert np.array_equal(y2, ref_y)
    st2 = cache.stats()
    if passes == 1:
        assert st2["misses"] == st["misses"] and st2["hits"] == st["hits"] + n
        assert st2["bytes_copied"] == st["bytes_copied"]
    cache.close()


@pytest.mark.timeout(300)
def test_cache_refuses_fp8_per_tensor_layers_that_need_several_passes():
    lay = _small("f8a8", 256, 8, 2, 256, "fp8", "fp8", 0)
    x = synth.make_tokens(lay, 64, stream=3)
    cache = ft.ExpertCache.from_host(lay, 2, DEV, path="prefill")
    with pytest.raises(ft.FtmoeError) as err:
        cache_forward(cache, x)
    assert err.value.status == ft.ERR_UNSUPPORTED
    cache.close()
