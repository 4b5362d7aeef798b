"""Python binding of libftmoe.so: the routed MoE layer forward over
block-quantised experts (MXFP4 / NVFP4 / FP8) on MI355X.

The binding only marshals arguments: every step of the forward runs in the
library's HIP kernels.  Tensors are torch device tensors (torch provides
device memory and streams); their pointers and the current HIP stream are
passed through the C ABI declared in ``include/ftmoe.h``.  Every entry point
fails loudly when the library has not been built; there is no fallback
implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libftmoe.so")

# ftmoe_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
# ftmoe_wfmt
W_MXFP4, W_NVFP4, W_FP8_E4M3, W_BF16 = 1, 2, 3, 4
# ftmoe_afmt
ACT_BF16, ACT_FP8_PER_TENSOR, ACT_MXFP8 = 0, 1, 2
# ftmoe_path
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2

FMT_CODES = {"mxfp4": W_MXFP4, "nvfp4": W_NVFP4, "fp8": W_FP8_E4M3, "bf16": W_BF16}
ACT_CODES = {"bf16": ACT_BF16, "fp8": ACT_FP8_PER_TENSOR, "mxfp8": ACT_MXFP8}
PATH_CODES = {"auto": PATH_AUTO, "decode": PATH_DECODE, "prefill": PATH_PREFILL}
BIAS_LOGITS, BIAS_SELECT = 0, 1
BIAS_CODES = {"logits": BIAS_LOGITS, "select": BIAS_SELECT}

# Every symbol include/ftmoe.h declares.
EXPORTS = (
    "ftmoe_workspace_bytes", "ftmoe_workspace_size", "ftmoe_align_max_padded", "ftmoe_align_workspace_size", "ftmoe_route",
    "ftmoe_align", "ftmoe_experts_forward", "ftmoe_forward", "ftmoe_quantize_fp8_per_tensor",
    "ftmoe_timing_enable", "ftmoe_timing_collect", "ftmoe_status_string", "ftmoe_last_error", "ftmoe_version",
    "ftmoe_packed_size", "ftmoe_pack_qweight", "ftmoe_cache_pool_size", "ftmoe_cache_create",
    "ftmoe_cache_destroy", "ftmoe_cache_plan", "ftmoe_cache_workspace_size", "ftmoe_cache_forward",
    "ftmoe_cache_stats", "ftmoe_cache_set_host_compute", "ftmoe_cache_host_stats", "ftmoe_host_expert_rows",
    "ftmoe_forward_noalloc",
)
ROLE_GATE_UP, ROLE_DOWN = 0, 1


class FtmoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class QWeightDesc(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
        ("codes", ctypes.c_void_p), ("block_scales", ctypes.c_void_p), ("tensor_scales", ctypes.c_void_p),
        ("packed", ctypes.c_void_p), ("row_scales", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("act", ctypes.c_int32), ("path", ctypes.c_int32),
        ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("gate_up", QWeightDesc), ("down", QWeightDesc),
        ("shared_inter", ctypes.c_int32), ("router_bias_mode", ctypes.c_int32),
        ("shared_gate_up", QWeightDesc), ("shared_down", QWeightDesc),
        ("shared_gate_w", ctypes.c_void_p),
    ]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libftmoe.so (once).  Raises if it is missing: build it with
    ``python -m block_scaled_fp4_router_amd.build``."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -m block_scaled_fp4_router_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    lib.ftmoe_workspace_size.argtypes = [P(LayerDesc), i32, P(sz)]
    lib.ftmoe_workspace_bytes.argtypes = [P(LayerDesc), i32]
    lib.ftmoe_workspace_bytes.restype = sz
    lib.ftmoe_align_max_padded.argtypes = [i32, i32, i32, i32]
    lib.ftmoe_align_max_padded.restype = i32
    lib.ftmoe_align_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.ftmoe_align_workspace_size.restype = sz
    lib.ftmoe_route.argtypes = [P(LayerDesc), vp, i32, vp, sz, vp, vp, vp, vp]
    lib.ftmoe_align.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ftmoe_experts_forward.argtypes = [P(LayerDesc), vp, i32, vp, vp, vp, vp, sz, vp, vp]
    lib.ftmoe_forward.argtypes = [P(LayerDesc), vp, i32, vp, sz, vp, vp, vp, vp]
    lib.ftmoe_forward_noalloc.argtypes = [P(LayerDesc), vp, i32, vp, vp, vp, vp]
    lib.ftmoe_quantize_fp8_per_tensor.argtypes = [vp, i64, vp, vp, vp, sz, vp]
    lib.ftmoe_packed_size.argtypes = [P(QWeightDesc), i32, P(sz)]
    lib.ftmoe_pack_qweight.argtypes = [P(QWeightDesc), i32, vp, sz, vp]
    lib.ftmoe_status_string.argtypes = [i32]
    lib.ftmoe_status_string.restype = ctypes.c_char_p
    lib.ftmoe_last_error.argtypes = []
    lib.ftmoe_last_error.restype = ctypes.c_char_p
    lib.ftmoe_version.restype = i32
    lib.ftmoe_timing_enable.argtypes = [i32]
    lib.ftmoe_timing_enable.restype = None
    lib.ftmoe_timing_collect.argtypes = [i32, ctypes.c_char_p, P(ctypes.c_double), P(i64)]
    lib.ftmoe_timing_collect.restype = i32
    lib.ftmoe_cache_pool_size.argtypes = [P(LayerDesc), i32, P(sz)]
    lib.ftmoe_cache_create.argtypes = [P(LayerDesc), P(QWeightDesc), P(QWeightDesc), i32, vp, sz, P(vp)]
    lib.ftmoe_cache_destroy.argtypes = [vp]
    lib.ftmoe_cache_destroy.restype = None
    lib.ftmoe_cache_plan.argtypes = [vp, vp, i32, vp, vp]
    lib.ftmoe_cache_workspace_size.argtypes = [vp, i32, P(sz)]
    lib.ftmoe_cache_forward.argtypes = [vp, vp, i32, vp, sz, vp, vp, vp, vp]
    lib.ftmoe_cache_stats.argtypes = [vp, P(i64), P(i64), P(i64), P(i64)]
    dbl = ctypes.c_double
    lib.ftmoe_cache_set_host_compute.argtypes = [vp, i32, dbl, dbl, dbl]
    lib.ftmoe_cache_host_stats.argtypes = [vp, P(i64), P(i64), P(dbl), P(dbl), P(dbl)]
    lib.ftmoe_host_expert_rows.argtypes = [P(LayerDesc), vp, vp, vp, i32, vp, i32]
    for name in ("ftmoe_workspace_size", "ftmoe_route", "ftmoe_align", "ftmoe_experts_forward",
                 "ftmoe_forward", "ftmoe_forward_noalloc", "ftmoe_quantize_fp8_per_tensor", "ftmoe_packed_size", "ftmoe_pack_qweight",
                 "ftmoe_cache_pool_size", "ftmoe_cache_create", "ftmoe_cache_plan", "ftmoe_cache_workspace_size",
                 "ftmoe_cache_forward", "ftmoe_cache_stats", "ftmoe_cache_set_host_compute",
                 "ftmoe_cache_host_stats", "ftmoe_host_expert_rows"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _status_name(st: int) -> str:
    try:
        return load().ftmoe_status_string(st).decode()
    except Exception:  # library missing: still say something useful
        return f"status {st}"


def _check(st: int) -> None:
    if st != OK:
        raise FtmoeError(st, load().ftmoe_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# --------------------------------------------------------------- layer ----


@dataclass
class DeviceQWeight:
    fmt: str
    num_experts: int
    n: int
    k: int
    codes: object
    block_scales: object = None
    tensor_scales: object = None
    packed: object = None   # the prefill tile layout (pack()), or None

    def desc(self) -> QWeightDesc:
        row_scales = 1 if self.tensor_scales is not None and self.tensor_scales.dim() == 2 else 0
        return QWeightDesc(FMT_CODES[self.fmt], self.num_experts, self.n, self.k, _ptr(self.codes),
                           _ptr(self.block_scales), _ptr(self.tensor_scales), _ptr(self.packed), row_scales, 0)

    def pack(self, role: int, stream=None) -> None:
        """Adds the prefill tile layout of these matrices (ftmoe_pack_qweight)."""
        import torch
        d = self.desc()
        d.packed = None
        n = ctypes.c_size_t(0)
        _check(load().ftmoe_packed_size(ctypes.byref(d), role, ctypes.byref(n)))
        buf = torch.empty(max(256, n.value), dtype=torch.uint8, device=self.codes.device)
        _check(load().ftmoe_pack_qweight(ctypes.byref(d), role, _ptr(buf), buf.numel(), _stream(stream)))
        self.packed = buf


class DeviceLayer:
    """A layer whose tensors live on the GPU, plus its C descriptor.

    ``from_host`` copies a host layer (numpy arrays with the attribute names
    of the generator's layers: router_w, router_b, gate_up, down, shared_*)
    to ``device``."""

    def __init__(self, hidden, inter, num_experts, top_k, router_w, gate_up: DeviceQWeight,
                 down: DeviceQWeight, router_bias=None, act="bf16", path="auto", shared_inter=0,
                 shared_gate_up: Optional[DeviceQWeight] = None, shared_down: Optional[DeviceQWeight] = None,
                 shared_gate_w=None, bias_mode="logits"):
        self.hidden, self.inter, self.num_experts, self.top_k = hidden, inter, num_experts, top_k
        self.router_w, self.router_bias, self.bias_mode = router_w, router_bias, bias_mode
        self.gate_up, self.down = gate_up, down
        self.act, self.path = act, path
        self.shared_inter = shared_inter
        self.shared_gate_up, self.shared_down, self.shared_gate_w = shared_gate_up, shared_down, shared_gate_w

    def pack(self) -> "DeviceLayer":
        """Adds the prefill tile layout of every matrix set (a load-time step;
        doubles the weights' footprint).  Returns self.  BF16 experts have
        no packed layout and are left as they are."""
        if self.gate_up.fmt == "bf16":
            return self
        self.gate_up.pack(ROLE_GATE_UP)
        self.down.pack(ROLE_DOWN)
        if self.shared_inter:
            self.shared_gate_up.pack(ROLE_GATE_UP)
            self.shared_down.pack(ROLE_DOWN)
        return self

    @classmethod
    def from_host(cls, lay, device="cuda", path="auto") -> "DeviceLayer":
        import numpy as np
        import torch

        def t(a):
            if a is None:
                return None
            if a.dtype == np.uint16:   # bf16 bit patterns travel as int16
                a = a.view(np.int16)
            return torch.from_numpy(a).to(device)

        def qw(q):
            if q is None:
                return None
            return DeviceQWeight(q.fmt, q.num_experts, q.n, q.k, t(q.codes), t(q.block_scales), t(q.tensor_scales))

        cfg = lay.cfg
        return cls(cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k, t(lay.router_w), qw(lay.gate_up),
                   qw(lay.down), router_bias=t(lay.router_b), act=cfg.act, path=path,
                   shared_inter=cfg.shared_inter, shared_gate_up=qw(lay.shared_gate_up),
                   shared_down=qw(lay.shared_down), shared_gate_w=t(lay.shared_gate_w),
                   bias_mode=getattr(cfg, "bias_mode", "logits"))

    def desc(self) -> LayerDesc:
        d = LayerDesc()
        d.hidden, d.inter, d.num_experts, d.top_k = self.hidden, self.inter, self.num_experts, self.top_k
        d.act, d.path = ACT_CODES[self.act], PATH_CODES[self.path]
        d.router_w, d.router_bias = _ptr(self.router_w), _ptr(self.router_bias)
        d.router_bias_mode = BIAS_CODES[self.bias_mode]
        d.gate_up, d.down = self.gate_up.desc(), self.down.desc()
        d.shared_inter = self.shared_inter
        if self.shared_inter:
            d.shared_gate_up, d.shared_down = self.shared_gate_up.desc(), self.shared_down.desc()
            d.shared_gate_w = _ptr(self.shared_gate_w)
        return d

    def with_path(self, path: str) -> "DeviceLayer":
        import copy
        c = copy.copy(self)
        c.path = path
        return c

    def selected_expert_bytes(self, ids) -> int:
        """Bytes of packed weights (codes + block scales + tensor scales) of
        the distinct experts in ``ids`` plus the shared expert."""
        import numpy as np
        u = np.unique(np.asarray(ids)).size

        def per_expert(q):
            b = q.codes[0].numel() * q.codes.element_size()
            if q.block_scales is not None:
                b += q.block_scales[0].numel()
            if q.tensor_scales is not None:
                b += q.tensor_scales[0].numel() * 4
            return b

        total = u * (per_expert(self.gate_up) + per_expert(self.down))
        if self.shared_inter:
            total += per_expert(self.shared_gate_up) + per_expert(self.shared_down)
        return total


# ----------------------------------------------------------- entry points --


def workspace_size(layer: DeviceLayer, T: int) -> int:
    n = ctypes.c_size_t(0)
    d = layer.desc()
    _check(load().ftmoe_workspace_size(ctypes.byref(d), T, ctypes.byref(n)))
    return n.value


def workspace_bytes(layer: DeviceLayer, T: int) -> int:
    """ftmoe_workspace_bytes: the same query as workspace_size, 0 on bad arguments."""
    d = layer.desc()
    return load().ftmoe_workspace_bytes(ctypes.byref(d), T)


def align_max_padded(T: int, k: int, E: int, block_m: int) -> int:
    return load().ftmoe_align_max_padded(T, k, E, block_m)


def align_workspace_size(T: int, k: int, E: int, block_m: int) -> int:
    return load().ftmoe_align_workspace_size(T, k, E, block_m)


def alloc_workspace(layer: DeviceLayer, T: int, device="cuda"):
    import torch
    n = max(256, workspace_size(layer, T))
    return torch.empty(n, dtype=torch.uint8, device=device)


def route(layer: DeviceLayer, x, T: int, ws, topk_ids, topk_w, shared_gate=None, stream=None) -> None:
    d = layer.desc()
    _check(load().ftmoe_route(ctypes.byref(d), _ptr(x), T, _ptr(ws), ws.numel(), _ptr(topk_ids), _ptr(topk_w),
                              _ptr(shared_gate), _stream(stream)))


def align(topk_ids, T: int, k: int, E: int, block_m: int, counts, offsets, sorted_ids, block_expert, num_padded,
          ws=None, stream=None) -> None:
    _check(load().ftmoe_align(_ptr(topk_ids), T, k, E, block_m, _ptr(counts), _ptr(offsets), _ptr(sorted_ids),
                              _ptr(block_expert), _ptr(num_padded), _ptr(ws), 0 if ws is None else ws.numel(),
                              _stream(stream)))


def experts_forward(layer: DeviceLayer, x, T: int, topk_ids, topk_w, shared_gate, ws, y, stream=None) -> None:
    d = layer.desc()
    _check(load().ftmoe_experts_forward(ctypes.byref(d), _ptr(x), T, _ptr(topk_ids), _ptr(topk_w),
                                        _ptr(shared_gate), _ptr(ws), ws.numel(), _ptr(y), _stream(stream)))


def forward(layer: DeviceLayer, x, T: int, ws, y, topk_ids=None, topk_w=None, stream=None, desc=None) -> None:
    d = desc if desc is not None else layer.desc()
    _check(load().ftmoe_forward(ctypes.byref(d), _ptr(x), T, _ptr(ws), ws.numel(), _ptr(y), _ptr(topk_ids),
                                _ptr(topk_w), _stream(stream)))


def forward_noalloc(layer: DeviceLayer, x, T: int, y, topk_ids=None, topk_w=None, stream=None, desc=None) -> None:
    """ftmoe_forward_noalloc: the layer forward on the library's own fixed
    scratch (no workspace, nothing allocated)."""
    d = desc if desc is not None else layer.desc()
    _check(load().ftmoe_forward_noalloc(ctypes.byref(d), _ptr(x), T, _ptr(y), _ptr(topk_ids), _ptr(topk_w),
                                        _stream(stream)))


class ExpertCache:
    """An HBM pool of ``slots`` expert slots over routed experts kept in host
    memory (ftmoe_cache_*).  ``layer`` is a DeviceLayer whose router and
    shared expert are used (its routed experts are not); ``host_gate_up``
    and ``host_down`` are DeviceQWeight-like holders of host tensors (pinned
    for asynchronous copies)."""

    def __init__(self, layer: DeviceLayer, host_gate_up: "DeviceQWeight", host_down: "DeviceQWeight", slots: int,
                 device="cuda"):
        import torch
        lib = load()
        self.layer, self.host_gate_up, self.host_down, self.slots = layer, host_gate_up, host_down, slots
        self._desc = layer.desc()
        n = ctypes.c_size_t(0)
        _check(lib.ftmoe_cache_pool_size(ctypes.byref(self._desc), slots, ctypes.byref(n)))
        self.pool = torch.empty(max(256, n.value), dtype=torch.uint8, device=device)
        self._hgu, self._hdn = host_gate_up.desc(), host_down.desc()
        h = ctypes.c_void_p(0)
        _check(lib.ftmoe_cache_create(ctypes.byref(self._desc), ctypes.byref(self._hgu), ctypes.byref(self._hdn),
                                      slots, _ptr(self.pool), self.pool.numel(), ctypes.byref(h)))
        self.handle = h

    @classmethod
    def from_host(cls, lay, slots: int, device="cuda", path="auto", pinned=True) -> "ExpertCache":
        """From a generator layer: router and shared expert on the device, the
        routed experts only in host memory (pinned unless ``pinned`` is
        False: the pool is then filled by staged DMA copies instead of the
        fill kernel)."""
        import numpy as np
        import torch

        def host(a):
            if a is None:
                return None
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            t = torch.from_numpy(np.ascontiguousarray(a))
            return t.pin_memory() if pinned else t.clone()

        def hq(q):
            return DeviceQWeight(q.fmt, q.num_experts, q.n, q.k, host(q.codes), host(q.block_scales),
                                 host(q.tensor_scales))

        gu, dn = hq(lay.gate_up), hq(lay.down)

        class _NoRouted:   # the layer without its routed experts, which stay on the host
            def __getattr__(self, name):
                return None if name in ("gate_up", "down") else getattr(lay, name)

        dl = DeviceLayer.from_host(_NoRouted(), device, path=path)
        dl.gate_up, dl.down = gu, dn   # descriptors only (the cache does not read a layer's routed experts)
        return cls(dl, gu, dn, slots, device)

    def plan(self, experts):
        """The residency policy alone (host): (slot per expert, miss flags)."""
        import numpy as np
        e = np.ascontiguousarray(experts, dtype=np.int32)
        sl = np.zeros(len(e), np.int32)
        miss = np.zeros(len(e), np.int32)
        _check(load().ftmoe_cache_plan(self.handle, e.ctypes.data, len(e), sl.ctypes.data, miss.ctypes.data))
        return sl, miss

    def workspace(self, T: int, device="cuda"):
        import torch
        n = ctypes.c_size_t(0)
        _check(load().ftmoe_cache_workspace_size(self.handle, T, ctypes.byref(n)))
        return torch.empty(max(256, n.value), dtype=torch.uint8, device=device)

    def forward(self, x, T: int, ws, y, topk_ids=None, topk_w=None, stream=None) -> None:
        _check(load().ftmoe_cache_forward(self.handle, _ptr(x), T, _ptr(ws), ws.numel(), _ptr(y), _ptr(topk_ids),
                                          _ptr(topk_w), _stream(stream)))

    def stats(self) -> dict:
        v = [ctypes.c_int64(0) for _ in range(4)]
        _check(load().ftmoe_cache_stats(self.handle, *[ctypes.byref(t) for t in v]))
        return dict(zip(("hits", "misses", "bytes_copied", "passes"), (t.value for t in v)))

    def set_host_compute(self, threads: int, expert_s: float = 0.0, row_s: float = -1.0,
                         link_bytes_per_s: float = 0.0) -> None:
        """CPU-GPU co-execution (ftmoe_cache_set_host_compute); expert_s <= 0
        or row_s < 0 calibrates the host cost model."""
        _check(load().ftmoe_cache_set_host_compute(self.handle, threads, expert_s, row_s, link_bytes_per_s))

    def host_stats(self) -> dict:
        i = [ctypes.c_int64(0) for _ in range(2)]
        d = [ctypes.c_double(0) for _ in range(3)]
        _check(load().ftmoe_cache_host_stats(self.handle, *[ctypes.byref(t) for t in i + d]))
        return dict(zip(("experts", "rows", "seconds", "expert_s", "row_s"), [t.value for t in i + d]))

    def close(self) -> None:
        if getattr(self, "handle", None):
            load().ftmoe_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def host_expert_rows(lay, x_bits, tok, ex, threads: int = 4):
    """The host half of co-execution alone (ftmoe_host_expert_rows), on a
    generator layer in host memory: o [n][H] fp32 for token tok[r] through
    routed expert ex[r]."""
    import numpy as np
    cfg = lay.cfg
    keep = []

    def arr(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a

    def qd(q):
        d = QWeightDesc()
        d.fmt, d.num_experts, d.n, d.k = FMT_CODES[q.fmt], q.num_experts, q.n, q.k
        d.codes = arr(q.codes).ctypes.data
        bs, ts = arr(q.block_scales), arr(q.tensor_scales)
        d.block_scales = bs.ctypes.data if bs is not None else None
        d.tensor_scales = ts.ctypes.data if ts is not None else None
        d.row_scales = 1 if ts is not None and ts.ndim == 2 else 0
        return d

    d = LayerDesc()
    d.hidden, d.inter, d.num_experts, d.top_k = cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k
    d.act, d.path = ACT_CODES[cfg.act], PATH_CODES["auto"]
    d.router_w = arr(lay.router_w).ctypes.data
    d.gate_up, d.down = qd(lay.gate_up), qd(lay.down)
    x = arr(np.asarray(x_bits, dtype=np.uint16))
    tok = arr(np.asarray(tok, dtype=np.int32))
    ex = arr(np.asarray(ex, dtype=np.int32))
    o = np.zeros((len(tok), cfg.hidden), np.float32)
    _check(load().ftmoe_host_expert_rows(ctypes.byref(d), x.ctypes.data, tok.ctypes.data, ex.ctypes.data, len(tok),
                                         o.ctypes.data, threads))
    return o


def quantize_fp8_per_tensor(x, n: int, q, scale, ws, stream=None) -> None:
    _check(load().ftmoe_quantize_fp8_per_tensor(_ptr(x), n, _ptr(q), _ptr(scale), _ptr(ws), ws.numel(),
                                                _stream(stream)))


def timing_enable(on: bool = True) -> None:
    """Bracket every kernel this thread enqueues with HIP events."""
    load().ftmoe_timing_enable(1 if on else 0)


def timing_collect(max_entries: int = 64) -> dict:
    """{kernel name: (total ms, launches)} since the last collect."""
    names = ctypes.create_string_buffer(32 * max_entries)
    ms = (ctypes.c_double * max_entries)()
    cnt = (ctypes.c_int64 * max_entries)()
    n = load().ftmoe_timing_collect(max_entries, names, ms, cnt)
    out = {}
    for i in range(min(n, max_entries)):
        name = names.raw[32 * i:32 * i + 32].split(b"\0", 1)[0].decode()
        out[name] = (ms[i], cnt[i])
    return out


def version() -> int:
    return load().ftmoe_version()
