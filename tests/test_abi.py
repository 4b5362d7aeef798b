"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and its host-side argument checks return the documented statuses
before anything touches a GPU (validation never dereferences the device
pointers, so placeholders stand in for them here)."""
import ctypes
import os
import re

import pytest

import block_scaled_fp4_router_amd as ft
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ftmoe.h")

needs_lib = pytest.mark.skipif(not os.path.exists(ft.LIB_PATH), reason="libftmoe.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ftmoe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("ftmoe_route", "ftmoe_align", "ftmoe_experts_forward", "ftmoe_forward"):
        assert n in names
    assert set(names) == set(ft.EXPORTS)


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ft.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


@needs_lib
@pytest.mark.parametrize("T,k,E,BM", [(0, 2, 8, 16), (1, 8, 128, 16), (8, 8, 128, 16), (16, 2, 8, 64),
                                      (4096, 8, 128, 64), (16384, 8, 128, 64), (37, 3, 5, 7)])
def test_align_capacity_matches_oracle(T, k, E, BM):
    assert ft.align_max_padded(T, k, E, BM) == oracle.align_max_padded(T, k, E, BM)


@needs_lib
def test_align_capacity_rejects_bad_sizes():
    for args in [(-1, 2, 8, 16), (4, 0, 8, 16), (4, 17, 32, 16), (4, 2, 0, 16), (4, 2, 8, 0), (4, 2, 2000, 16)]:
        assert ft.align_max_padded(*args) == -1


FAKE = 1 << 20  # an aligned placeholder address; never dereferenced by validation


def _qw(fmt, E, n, k):
    return ft.QWeightDesc(fmt, E, n, k, FAKE, FAKE, FAKE)


def good_layer():
    d = ft.LayerDesc()
    d.hidden, d.inter, d.num_experts, d.top_k = 256, 128, 8, 2
    d.act, d.path = ft.ACT_BF16, ft.PATH_AUTO
    d.router_w, d.router_bias = FAKE, None
    d.gate_up = _qw(ft.W_MXFP4, 8, 256, 256)
    d.down = _qw(ft.W_MXFP4, 8, 256, 128)
    return d


def _ws_status(d, T=16):
    n = ctypes.c_size_t(0)
    return ft.load().ftmoe_workspace_size(ctypes.byref(d), T, ctypes.byref(n)), n.value


@needs_lib
def test_workspace_size_of_a_valid_layer():
    st, n = _ws_status(good_layer())
    assert st == ft.OK and n > 0 and n % 256 == 0


@needs_lib
@pytest.mark.parametrize("field,value,status", [
    ("hidden", 100, ft.ERR_UNSUPPORTED),
    ("hidden", 4096 + 128, ft.ERR_UNSUPPORTED),
    ("inter", 192, ft.ERR_UNSUPPORTED),
    ("inter", 4096 + 128, ft.ERR_UNSUPPORTED),
    ("inter", 0, ft.ERR_UNSUPPORTED),
    ("top_k", 0, ft.ERR_UNSUPPORTED),
    ("top_k", 9, ft.ERR_UNSUPPORTED),
    ("num_experts", 2000, ft.ERR_UNSUPPORTED),
    ("act", 7, ft.ERR_INVALID_ARG),
    ("router_bias_mode", 2, ft.ERR_INVALID_ARG),
    ("path", 9, ft.ERR_INVALID_ARG),
    ("router_w", None, ft.ERR_INVALID_ARG),
    ("router_w", FAKE + 4, ft.ERR_INVALID_ARG),
    ("act", ft.ACT_FP8_PER_TENSOR, ft.ERR_UNSUPPORTED),   # FP8 activations need FP8 weights
])
def test_layer_validation(field, value, status):
    d = good_layer()
    setattr(d, field, value)
    assert _ws_status(d)[0] == status
    assert ft.load().ftmoe_last_error().decode() != ""


@needs_lib
def test_mxfp8_activations_need_mxfp4_weights_and_shrink_the_workspace():
    d = good_layer()
    _, n_split = _ws_status(d, T=8)
    _, n_split_pf = _ws_status(d, T=4096)
    d.act = ft.ACT_MXFP8
    st, n8 = _ws_status(d, T=8)
    st_pf, n8_pf = _ws_status(d, T=4096)
    assert st == ft.OK and st_pf == ft.OK
    # no lo code plane: decode drops T*H (x) and the h rows' bytes, prefill T*H
    assert n8 < n_split and n8_pf < n_split_pf
    for fmt in (ft.W_NVFP4, ft.W_FP8_E4M3):
        d2 = good_layer()
        d2.act = ft.ACT_MXFP8
        d2.gate_up = _qw(fmt, 8, 256, 256)
        d2.down = _qw(fmt, 8, 256, 128)
        assert _ws_status(d2)[0] == ft.ERR_UNSUPPORTED
        assert "MXFP8" in ft.load().ftmoe_last_error().decode()


@needs_lib
def test_weight_shape_and_format_validation():
    d = good_layer()
    d.down = _qw(ft.W_MXFP4, 8, 256, 256)          # K must equal inter
    assert _ws_status(d)[0] == ft.ERR_INVALID_ARG
    d = good_layer()
    d.down = _qw(ft.W_NVFP4, 8, 256, 128)          # mixed formats
    assert _ws_status(d)[0] == ft.ERR_INVALID_ARG
    d = good_layer()
    d.gate_up.block_scales = None
    assert _ws_status(d)[0] == ft.ERR_INVALID_ARG
    d = good_layer()
    d.gate_up.fmt = d.down.fmt = 9
    assert _ws_status(d)[0] == ft.ERR_INVALID_ARG
    d = good_layer()
    d.shared_inter = 128                           # shared expert without its tensors
    d.shared_gate_up = ft.QWeightDesc(ft.W_MXFP4, 1, 256, 256, None, None, None)
    assert _ws_status(d)[0] == ft.ERR_INVALID_ARG


@needs_lib
def test_bf16_experts_validation():
    d = good_layer()
    d.gate_up = _qw(ft.W_BF16, 8, 256, 256)
    d.down = _qw(ft.W_BF16, 8, 256, 128)
    assert _ws_status(d)[0] == ft.OK
    d.gate_up.row_scales = 1                       # no fp32 multipliers
    assert _ws_status(d)[0] == ft.ERR_INVALID_ARG
    d.gate_up.row_scales = 0
    d.act = ft.ACT_FP8_PER_TENSOR                  # bf16 activations only
    assert _ws_status(d)[0] == ft.ERR_UNSUPPORTED
    d.act = ft.ACT_BF16
    d.gate_up.packed = FAKE                        # no packed layout
    assert _ws_status(d)[0] == ft.ERR_INVALID_ARG
    n = ctypes.c_size_t(0)
    assert ft.load().ftmoe_packed_size(ctypes.byref(_qw(ft.W_BF16, 8, 256, 256)), ft.ROLE_GATE_UP,
                                       ctypes.byref(n)) == ft.ERR_UNSUPPORTED


@needs_lib
def test_row_scale_flag_validation():
    d = good_layer()
    d.gate_up.row_scales = 1                       # MXFP4 has no fp32 multipliers
    assert _ws_status(d)[0] == ft.ERR_INVALID_ARG
    for fmt in (ft.W_NVFP4, ft.W_FP8_E4M3):
        d = good_layer()
        d.gate_up = _qw(fmt, 8, 256, 256)
        d.down = _qw(fmt, 8, 256, 128)
        d.gate_up.row_scales = 1
        assert _ws_status(d)[0] == ft.OK
        d.down.row_scales = 2
        assert _ws_status(d)[0] == ft.ERR_INVALID_ARG
        d.down.row_scales = 0
        d.down.reserved = 1
        assert _ws_status(d)[0] == ft.ERR_INVALID_ARG


@needs_lib
def test_tokens_and_workspace_validation():
    d = good_layer()
    lib = ft.load()
    assert _ws_status(d, T=-1)[0] == ft.ERR_INVALID_ARG
    n = _ws_status(d, T=16)[1]
    # too small a workspace is refused before anything is enqueued
    st = lib.ftmoe_forward(ctypes.byref(d), FAKE, 16, FAKE, n - 256, FAKE, None, None, None)
    assert st == ft.ERR_WORKSPACE
    st = lib.ftmoe_forward(ctypes.byref(d), FAKE, 16, FAKE + 16, n, FAKE, None, None, None)
    assert st == ft.ERR_WORKSPACE                  # not 256-byte aligned
    st = lib.ftmoe_forward(ctypes.byref(d), None, 16, FAKE, n, FAKE, None, None, None)
    assert st == ft.ERR_INVALID_ARG
    st = lib.ftmoe_forward(ctypes.byref(d), FAKE + 2, 16, FAKE, n, FAKE, None, None, None)
    assert st == ft.ERR_INVALID_ARG                # misaligned x
    # T = 0 is a valid no-op that touches nothing
    assert lib.ftmoe_forward(ctypes.byref(d), None, 0, None, 0, None, None, None, None) == ft.OK


@needs_lib
def test_shared_expert_needs_gate_output():
    d = good_layer()
    d.shared_inter = 128
    d.shared_gate_up = _qw(ft.W_MXFP4, 1, 256, 256)
    d.shared_down = _qw(ft.W_MXFP4, 1, 256, 128)
    d.shared_gate_w = FAKE
    st, n = _ws_status(d)
    assert st == ft.OK
    lib = ft.load()
    assert lib.ftmoe_route(ctypes.byref(d), FAKE, 16, FAKE, n, FAKE, FAKE, None, None) == ft.ERR_INVALID_ARG
    assert lib.ftmoe_experts_forward(ctypes.byref(d), FAKE, 16, FAKE, FAKE, None, FAKE, n, FAKE,
                                     None) == ft.ERR_INVALID_ARG


@needs_lib
def test_align_validation():
    lib = ft.load()
    assert lib.ftmoe_align(None, 4, 2, 8, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == ft.ERR_INVALID_ARG
    assert lib.ftmoe_align(FAKE, 4, 2, 8, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == ft.ERR_INVALID_ARG
    need = ft.align_workspace_size(4096, 8, 128, 64)
    assert need > 0
    assert lib.ftmoe_align(FAKE, 4096, 8, 128, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 4,
                           None) == ft.ERR_WORKSPACE


@needs_lib
def test_status_strings():
    lib = ft.load()
    assert lib.ftmoe_status_string(ft.ERR_WORKSPACE) == b"FTMOE_ERR_WORKSPACE"
    assert lib.ftmoe_status_string(99) == b"FTMOE_UNKNOWN_STATUS"
    assert ft.version() >= 100


@needs_lib
@pytest.mark.parametrize("fmt,E,n,k,role,stage", [
    (ft.W_MXFP4, 8, 256, 256, ft.ROLE_GATE_UP, 512 * 32 + 512 * 4),
    (ft.W_MXFP4, 128, 1536, 2048, ft.ROLE_GATE_UP, 512 * 32 + 512 * 4),
    (ft.W_MXFP4, 128, 2048, 768, ft.ROLE_DOWN, 512 * 32 + 512 * 4),
    (ft.W_NVFP4, 512, 1024, 2048, ft.ROLE_GATE_UP, 512 * 32 + 512 * 4),
    (ft.W_FP8_E4M3, 128, 3072, 4096, ft.ROLE_GATE_UP, 512 * 64),
    (ft.W_FP8_E4M3, 128, 4096, 1536, ft.ROLE_DOWN, 512 * 64),
])
def test_packed_size(fmt, E, n, k, role, stage):
    """E experts x tiles of 512 rows (gate_up: 256 gate + 256 up) x K/64 stages."""
    tiles = -(-(n // 2) // 256) if role == ft.ROLE_GATE_UP else -(-n // 512)
    q = ft.QWeightDesc(fmt, E, n, k, FAKE, FAKE, FAKE, None)
    got = ctypes.c_size_t(0)
    assert ft.load().ftmoe_packed_size(ctypes.byref(q), role, ctypes.byref(got)) == ft.OK
    assert got.value == E * tiles * (k // 64) * stage


@needs_lib
def test_packed_size_rejects_bad_arguments():
    lib = ft.load()
    got = ctypes.c_size_t(0)
    q = ft.QWeightDesc(ft.W_MXFP4, 8, 256, 256, FAKE, FAKE, FAKE, None)
    assert lib.ftmoe_packed_size(ctypes.byref(q), 7, ctypes.byref(got)) == ft.ERR_INVALID_ARG
    q.k = 100
    assert lib.ftmoe_packed_size(ctypes.byref(q), ft.ROLE_DOWN, ctypes.byref(got)) == ft.ERR_UNSUPPORTED
    q.k, q.fmt = 256, 9
    assert lib.ftmoe_packed_size(ctypes.byref(q), ft.ROLE_DOWN, ctypes.byref(got)) == ft.ERR_INVALID_ARG
    q.fmt = ft.W_MXFP4
    # misaligned destination, and too small a destination, are refused before any launch
    assert lib.ftmoe_pack_qweight(ctypes.byref(q), ft.ROLE_DOWN, FAKE + 16, 1 << 30, None) == ft.ERR_INVALID_ARG
    assert lib.ftmoe_pack_qweight(ctypes.byref(q), ft.ROLE_DOWN, FAKE, 16, None) == ft.ERR_INVALID_ARG


@needs_lib
def test_layer_rejects_misaligned_packed_weights():
    d = good_layer()
    d.gate_up.packed = FAKE + 16
    assert _ws_status(d)[0] == ft.ERR_INVALID_ARG


# ---- expert residency: the LRU policy (host only) ----
def _cache(slots, E=8):
    d = good_layer()
    d.num_experts = E
    d.gate_up = _qw(ft.W_MXFP4, E, 256, 256)
    d.down = _qw(ft.W_MXFP4, E, 256, 128)
    lib = ft.load()
    n = ctypes.c_size_t(0)
    assert lib.ftmoe_cache_pool_size(ctypes.byref(d), slots, ctypes.byref(n)) == ft.OK
    # 256-aligned regions; per slot: gate_up 256*256/2 + 256*256/32, down 256*128/2 + 256*128/32; then the
    # residency table of E int32 rounded up to 256 bytes
    assert n.value == slots * (256 * 256 // 2) + slots * (256 * 256 // 32) + slots * (256 * 128 // 2) + \
        slots * (256 * 128 // 32) + (E * 4 + 255) // 256 * 256
    h = ctypes.c_void_p(0)
    gu, dn = _qw(ft.W_MXFP4, E, 256, 256), _qw(ft.W_MXFP4, E, 256, 128)
    assert lib.ftmoe_cache_create(ctypes.byref(d), ctypes.byref(gu), ctypes.byref(dn), slots, FAKE, n.value,
                                  ctypes.byref(h)) == ft.OK
    return h


class _LRU:
    """The policy written out: an expert holding a slot keeps it; the others
    take free slots by (last use, slot index), never used first.  A plan on
    its own copies nothing, so every expert it lists still has to be copied
    (a miss) until a forward fills its slot; the slots are the same either
    way."""

    def __init__(self, slots):
        self.slot_of, self.exp_of, self.last, self.clock = {}, [None] * slots, [-1] * slots, 0

    def plan(self, experts):
        needed = {self.slot_of[e] for e in experts if e in self.slot_of}
        free = sorted((s for s in range(len(self.exp_of)) if s not in needed), key=lambda s: (self.last[s], s))
        self.clock += 1
        out = []
        for e in experts:
            if e in self.slot_of:
                s = self.slot_of[e]
            else:
                s = free.pop(0)
                if self.exp_of[s] is not None:
                    del self.slot_of[self.exp_of[s]]
                self.exp_of[s], self.slot_of[e] = e, s
            self.last[s] = self.clock
            out.append((s, 1))
        return out


@needs_lib
def test_cache_plan_is_lru():
    import numpy as np
    lib = ft.load()
    h = _cache(slots=4, E=8)
    model = _LRU(4)
    rng = np.random.default_rng(4)
    steps = [[0, 1, 2], [1, 3], [4, 5], [0, 6, 7, 1], [2], [2, 3, 4, 5]]
    steps += [sorted(rng.choice(8, size=rng.integers(1, 5), replace=False).tolist()) for _ in range(40)]
    hits = misses = 0
    for st in steps:
        e = np.array(st, np.int32)
        sl, miss = np.zeros(len(e), np.int32), np.zeros(len(e), np.int32)
        assert lib.ftmoe_cache_plan(h, e.ctypes.data, len(e), sl.ctypes.data, miss.ctypes.data) == ft.OK
        ref = model.plan(st)
        assert [(int(a), int(b)) for a, b in zip(sl, miss)] == ref
        assert len(set(sl.tolist())) == len(sl)       # distinct slots within a step
        hits += int((miss == 0).sum())
        misses += int(miss.sum())
    v = [ctypes.c_int64(0) for _ in range(4)]
    assert lib.ftmoe_cache_stats(h, *[ctypes.byref(t) for t in v]) == ft.OK
    assert (v[0].value, v[1].value) == (hits, misses)
    # too many experts for the slots, a repeated expert, or one out of range: refused, state unchanged
    for bad, status in (([0, 1, 2, 3, 4], ft.ERR_UNSUPPORTED), ([1, 1], ft.ERR_INVALID_ARG),
                        ([9], ft.ERR_INVALID_ARG)):
        e = np.array(bad, np.int32)
        assert lib.ftmoe_cache_plan(h, e.ctypes.data, len(e), None, None) == status
    lib.ftmoe_cache_destroy(h)


# The boundary's contract: the names and C signatures of the layer entry
# points.  Two documented deviations add caller scratch to ftmoe_route and
# ftmoe_align (the library never allocates device memory), marked "+ws".
CONTRACT = {
    "ftmoe_workspace_bytes": ("size_t", ["const ftmoe_layer*", "int32_t"]),
    "ftmoe_align_max_padded": ("int32_t", ["int32_t", "int32_t", "int32_t", "int32_t"]),
    "ftmoe_route": ("ftmoe_status", ["const ftmoe_layer*", "const uint16_t*", "int32_t", "+ws", "int32_t*",
                                     "float*", "float*", "void*"]),
    "ftmoe_align": ("ftmoe_status", ["const int32_t*", "int32_t", "int32_t", "int32_t", "int32_t", "int32_t*",
                                     "int32_t*", "int32_t*", "int32_t*", "int32_t*", "+ws", "void*"]),
    "ftmoe_experts_forward": ("ftmoe_status", ["const ftmoe_layer*", "const uint16_t*", "int32_t",
                                               "const int32_t*", "const float*", "const float*", "void*", "size_t",
                                               "uint16_t*", "void*"]),
    "ftmoe_forward": ("ftmoe_status", ["const ftmoe_layer*", "const uint16_t*", "int32_t", "void*", "size_t",
                                       "uint16_t*", "int32_t*", "float*", "void*"]),
    "ftmoe_status_string": ("const char*", ["ftmoe_status"]),
}


def header_prototypes():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"([A-Za-z_][A-Za-z0-9_ ]*?\s*\*?)\s*\b(ftmoe_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        ret = " ".join(m.group(1).replace("*", " * ").split()).replace(" *", "*")
        params = []
        for p in m.group(3).split(","):
            p = " ".join(p.replace("*", " * ").split())
            if not p or p == "void":
                continue
            words = p.split(" ")
            # drop the parameter name (the last word unless it is part of the type)
            if words[-1] not in ("*",) and len(words) > 1 and words[-1] not in ("int32_t", "size_t", "float"):
                words = words[:-1]
            params.append(" ".join(words).replace(" *", "*"))
        out[m.group(2)] = (ret, params)
    return out


def test_contract_names_and_signatures():
    protos = header_prototypes()
    for name, (ret, params) in CONTRACT.items():
        assert name in protos, name
        got_ret, got = protos[name]
        assert got_ret == ret, (name, got_ret)
        want = []
        for p in params:
            want += ["void*", "size_t"] if p == "+ws" else [p]
        assert got == want, (name, got)


@needs_lib
def test_workspace_bytes_matches_workspace_size():
    lib = ft.load()
    d = good_layer()
    for T in (0, 1, 8, 16, 17, 4096):
        n = ctypes.c_size_t(0)
        assert lib.ftmoe_workspace_size(ctypes.byref(d), T, ctypes.byref(n)) == ft.OK
        assert lib.ftmoe_workspace_bytes(ctypes.byref(d), T) == n.value > 0
    assert lib.ftmoe_workspace_bytes(ctypes.byref(d), -1) == 0
    assert lib.ftmoe_workspace_bytes(None, 4) == 0
    d.hidden = 100
    assert lib.ftmoe_workspace_bytes(ctypes.byref(d), 4) == 0
    assert b"hidden" in lib.ftmoe_last_error()


@needs_lib
def test_noalloc_forward_rejects_what_its_scratch_cannot_hold():
    """The allocation-free forward checks its fixed scratch before touching
    the GPU: a batch whose workspace exceeds it is refused with a message."""
    lib = ft.load()
    d = good_layer()
    n = ctypes.c_size_t(0)
    T = 1 << 20
    assert lib.ftmoe_workspace_size(ctypes.byref(d), T, ctypes.byref(n)) == ft.OK
    assert n.value > 32 << 20
    assert lib.ftmoe_forward_noalloc(ctypes.byref(d), FAKE, T, FAKE, None, None, None) == ft.ERR_WORKSPACE
    assert b"scratch" in lib.ftmoe_last_error()
    assert lib.ftmoe_forward_noalloc(ctypes.byref(d), None, 4, FAKE, None, None, None) == ft.ERR_INVALID_ARG
    assert lib.ftmoe_forward_noalloc(ctypes.byref(d), FAKE, 0, FAKE, None, None, None) == ft.OK   # empty batch


@needs_lib
@pytest.mark.parametrize("fmt,act", [("W_MXFP4", "ACT_BF16"), ("W_MXFP4", "ACT_MXFP8"), ("W_NVFP4", "ACT_BF16"),
                                     ("W_FP8_E4M3", "ACT_FP8_PER_TENSOR"), ("W_BF16", "ACT_BF16")])
def test_noalloc_scratch_holds_eight_token_decode_at_the_largest_shapes(fmt, act):
    """The header's promise for the allocation-free forward: an 8-token
    batch fits its 32 MiB scratch at hidden = intermediate = 4096, 1024
    experts, top-16 (and a 16-token one there does not)."""
    lib = ft.load()
    H = I = 4096
    E, k = 1024, 16
    d = ft.LayerDesc()
    d.hidden, d.inter, d.num_experts, d.top_k = H, I, E, k
    d.act, d.path = getattr(ft, act), ft.PATH_AUTO
    d.router_w, d.router_bias = FAKE, None
    d.gate_up = _qw(getattr(ft, fmt), E, 2 * I, H)
    d.down = _qw(getattr(ft, fmt), E, H, I)
    assert 0 < lib.ftmoe_workspace_bytes(ctypes.byref(d), 8) <= 32 << 20
    n16 = lib.ftmoe_workspace_bytes(ctypes.byref(d), 16)
    assert n16 > 0
    if n16 > 32 << 20:
        assert lib.ftmoe_forward_noalloc(ctypes.byref(d), FAKE, 16, FAKE, None, None, None) == ft.ERR_WORKSPACE
