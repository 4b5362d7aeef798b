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
import oracle
import synth
from gpu_util import DEV, bf16_dev_to_f64, layer_pair, rel_fro, run_forward, say, to_dev_bf16

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


class _PoolModel:
    """The residency policy the library documents, replayed on the host: per
    step, the resident experts form the first pass (run at once on the
    device's residency table, so it exists even when empty) and the missing
    ones follow (one pass if they fit beside them, else groups of half the
    pool; one pass of everything for per-tensor FP8 activations); each pass
    gives a missing expert the least recently used slot the pass does not
    need."""

    def __init__(self, E, slots, fp8=False):
        self.slots, self.fp8 = slots, fp8
        self.slot_of = {}
        self.owner = [-1] * slots
        self.last = [-1] * slots
        self.clock = 0
        self.hits = self.misses = self.passes = 0

    def _plan(self, group):
        needed = {self.slot_of[e] for e in group if e in self.slot_of}
        cand = sorted((s for s in range(self.slots) if s not in needed), key=lambda s: self.last[s])
        self.clock += 1
        nxt = 0
        for e in group:
            if e in self.slot_of:
                self.hits += 1
                s = self.slot_of[e]
            else:
                self.misses += 1
                s = cand[nxt]
                nxt += 1
                if self.owner[s] >= 0:
                    del self.slot_of[self.owner[s]]
                self.owner[s] = e
                self.slot_of[e] = s
            self.last[s] = self.clock

    def step(self, experts):
        experts = sorted(int(e) for e in experts)
        hit = [e for e in experts if e in self.slot_of]
        miss = [e for e in experts if e not in self.slot_of]
        if self.fp8:
            groups = [hit + miss]
        else:
            groups = [hit]
            g = max(1, len(miss)) if len(experts) <= self.slots else max(1, self.slots // 2)
            groups += [miss[a:a + g] for a in range(0, len(miss), g)]
        for grp in groups:
            self._plan(grp)
        self.passes += len(groups)

    def stats(self):
        return {"hits": self.hits, "misses": self.misses, "passes": self.passes}


CASES = [
    # name, layer, T, path, slots[, host memory pinned]
    ("c1", None, 8, "decode", 64),
    ("c1", None, 8, "decode", 12, False),
    ("c1", None, 8, "decode", 12),
    ("c1", None, 8, "decode", 1),
    ("c1-w4a8", None, 8, "decode", 20),
    ("c1", None, 40, "prefill", 24),
    ("nvs", (256, 16, 4, 128, "nvfp4", "bf16", 128), 9, "decode", 5),
    ("nvs", (256, 16, 4, 128, "nvfp4", "bf16", 128), 70, "prefill", 5),
    ("f8a8", (256, 8, 2, 256, "fp8", "fp8", 0), 12, "decode", 8),
    ("f8a8", (256, 8, 2, 256, "fp8", "fp8", 0), 300, "prefill", 8),
    ("bf16", (256, 8, 2, 256, "bf16", "bf16", 0), 70, "prefill", 3),
]


@pytest.mark.parametrize("name,shape,T,path,slots,pinned", [c if len(c) == 6 else c + (True,) for c in CASES])
@pytest.mark.timeout(600)
def test_cache_forward_equals_device_layer(name, shape, T, path, slots, pinned):
    say(f"expert cache {name} T={T} path={path} slots={slots} pinned={pinned}")
    if shape is None:
        lay, dlay = layer_pair(name)
    else:
        lay = _small(name, *shape)
        dlay = ft.DeviceLayer.from_host(lay, DEV)
    x = synth.make_tokens(lay, T, stream=T)
    ref_y, ref_ids, ref_w = run_forward(dlay, x, path)
    cache = ft.ExpertCache.from_host(lay, slots, DEV, path=path, pinned=pinned)
    y, ids, w = cache_forward(cache, x)
    assert np.array_equal(ids, ref_ids) and np.array_equal(w, ref_w)
    assert np.array_equal(y, ref_y)
    per_expert = sum(t.numel() * t.element_size() for t in (cache.host_gate_up.codes, cache.host_gate_up.block_scales,
                                                           cache.host_gate_up.tensor_scales, cache.host_down.codes,
                                                           cache.host_down.block_scales,
                                                           cache.host_down.tensor_scales) if t is not None) // dlay.num_experts
    model = _PoolModel(dlay.num_experts, slots, fp8=lay.cfg.act == "fp8")
    step = np.unique(ids)
    model.step(step)
    st = cache.stats()
    say(f"  distinct experts {len(step)}, stats {st}, model {model.stats()}")
    assert st == dict(model.stats(), bytes_copied=model.misses * per_expert)
    # the same step again: the experts that stayed resident are hits and run first
    y2, ids2, _ = cache_forward(cache, x)
    assert np.array_equal(y2, ref_y)
    model.step(step)
    st2 = cache.stats()
    say(f"  second step: stats {st2}")
    assert st2 == dict(model.stats(), bytes_copied=model.misses * per_expert)
    if len(step) <= slots:
        assert st2["misses"] == st["misses"] and st2["passes"] == st["passes"] + 1
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


# ------------------------------------------------------------ co-execution --
HOST_CASES = [
    # name, layer, T, path, slots, mode: "all" (every miss on the host), "none", "calibrated"
    ("c1", None, 8, "decode", 12, "all"),
    ("c1", None, 8, "decode", 12, "none"),
    ("c1", None, 8, "decode", 24, "calibrated"),
    ("c1-w4a8", None, 8, "decode", 20, "all"),
    ("c1", None, 40, "prefill", 24, "all"),
    ("nvs", (256, 16, 4, 128, "nvfp4", "bf16", 128), 70, "prefill", 5, "all"),
    ("bf16", (256, 8, 2, 256, "bf16", "bf16", 0), 9, "decode", 3, "all"),
]


@pytest.mark.parametrize("name,shape,T,path,slots,mode", HOST_CASES)
@pytest.mark.timeout(600)
def test_cache_host_compute(name, shape, T, path, slots, mode):
    """Missing experts computed on the host cores: the layer output stays
    within 1e-2 of the device-only output (relative Frobenius; the host
    sums in another order) and within the layer's tolerance of the oracle;
    the routing is unchanged; the counters add up."""
    say(f"expert cache + host compute {name} T={T} path={path} slots={slots} mode={mode}")
    if shape is None:
        lay, dlay = layer_pair(name)
    else:
        lay = _small(name, *shape)
        dlay = ft.DeviceLayer.from_host(lay, DEV)
    x = synth.make_tokens(lay, T, stream=T + 1)
    ref_y, ref_ids, ref_w = run_forward(dlay, x, path)
    cache = ft.ExpertCache.from_host(lay, slots, DEV, path=path)
    if mode == "all":
        cache.set_host_compute(4, expert_s=1e-12, row_s=0.0, link_bytes_per_s=1.0)
    elif mode == "none":
        cache.set_host_compute(4, expert_s=1e3, row_s=0.0)
    else:
        cache.set_host_compute(4)
    hs0 = cache.host_stats()
    say(f"  cost model {hs0}")
    assert hs0["expert_s"] > 0 and hs0["row_s"] >= 0
    for step in range(2):
        y, ids, w = cache_forward(cache, x)
        assert np.array_equal(ids, ref_ids) and np.array_equal(w, ref_w)
        assert np.isfinite(y).all()
        err = rel_fro(y, ref_y)
        say(f"  step {step}: vs device-only {err:.2e}, pool {cache.stats()}, host {cache.host_stats()}")
        assert err <= 1e-2
        if mode == "none":
            assert np.array_equal(y, ref_y)
    hs, st = cache.host_stats(), cache.stats()
    n = len(np.unique(ids))
    if mode == "all":
        # nothing is ever resident: every expert of both steps is computed on the host
        assert hs["experts"] == 2 * n and hs["rows"] == 2 * ids.size
        assert st["hits"] == 0 and st["misses"] == 0 and st["bytes_copied"] == 0
    elif mode == "none":
        assert hs["experts"] == 0 and hs["rows"] == 0
    else:
        assert hs["experts"] + st["hits"] + st["misses"] == 2 * n
    tok = np.arange(T)
    s_h = None
    ref = oracle.forward_tokens(lay, x, tok, s_h=s_h)
    err = rel_fro(y, ref)
    say(f"  vs oracle {err:.2e}")
    assert err <= (3e-2 if lay.cfg.act in ("fp8", "mxfp8") else 2e-2)
    cache.close()


@pytest.mark.timeout(300)
def test_host_compute_refuses_fp8_per_tensor_layers():
    lay = _small("f8a8", 256, 8, 2, 256, "fp8", "fp8", 0)
    cache = ft.ExpertCache.from_host(lay, 8, DEV, path="decode")
    with pytest.raises(ft.FtmoeError) as err:
        cache.set_host_compute(2)
    assert err.value.status == ft.ERR_UNSUPPORTED
    cache.close()


@pytest.mark.parametrize("path,T", [("decode", 8), ("prefill", 40)])
@pytest.mark.timeout(600)
def test_plan_then_forward_equals_device_layer(path, T):
    """A plan on its own (ftmoe_cache_plan) copies nothing: the experts it
    places, and the ones it evicts, must not count as resident in the next
    forward, whose output stays bit-equal to the device layer's."""
    say(f"expert cache plan then forward c1 T={T} path={path}")
    lay, dlay = layer_pair("c1")
    xa = synth.make_tokens(lay, T, stream=41)
    xb = synth.make_tokens(lay, T, stream=42)
    cache = ft.ExpertCache.from_host(lay, 48, DEV, path=path)
    ya, ids_a, _ = cache_forward(cache, xa)            # fills the pool with step a's experts
    ref_b = run_forward(dlay, xb, path)
    ids_b = ref_b[1]
    # plan b's experts, and then a's again (evicting some of b's placements
    # and re-placing a's resident experts), without any copy
    eb = np.unique(ids_b)
    ea = np.unique(ids_a)
    cache.plan(eb[:40])
    sl, miss = cache.plan(ea[:40])
    assert miss.sum() >= 0
    yb, idsb, wb = cache_forward(cache, xb)
    assert np.array_equal(idsb, ids_b) and np.array_equal(wb, ref_b[2])
    assert np.array_equal(yb, ref_b[0]), "pool forward after a plan differs from the device layer"
    ya2, _, _ = cache_forward(cache, xa)
    assert np.array_equal(ya2, ya)
