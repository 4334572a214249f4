"""ctypes binding of libmoe_gfx950.so (argument marshalling only).

Every step of the layer runs in the library's HIP kernels; torch is used here
only to allocate device / pinned memory and to name the current stream.  If
the shared library is missing this module raises at import: there is no
fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gfx950.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("routed_expert_cache_amd: %s is not built; run "
                      "`python -m routed_expert_cache_amd.build` (hipcc, gfx950)" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_ARG", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_NO_SPACE",
          -4: "MOE_ERR_NOT_PINNED", -5: "MOE_ERR_HIP", -6: "MOE_ERR_STATE", -7: "MOE_ERR_DEVICE"}
W_BF16, W_FP8_B128 = 0, 1
STEP_NO_COPY = 1
STEP_FILL_ALL = 2
HOST_PORTABLE = 1
HOST_PIN = 2
FWD_DECODE, FWD_PREFILL, FWD_DECODE_SPLIT = 0, 1, 2
CNT_UNIQ, CNT_HIT, CNT_MISS, CNT_QSTAR, CNT_FILL, CNT_HOST, CNT_N = 0, 1, 2, 3, 4, 5, 8

EXPORTS = [
    "moe_last_error", "moe_route_topk", "moe_cache_workspace_bytes", "moe_cache_create",
    "moe_cache_seed", "moe_cache_step", "moe_cache_route_step", "moe_cache_fill", "moe_cache_read_state", "moe_cache_error",
    "moe_cache_destroy", "moe_forward_workspace_bytes", "moe_expert_forward", "moe_expert_forward_merge",
    "moe_expert_forward_merge_static", "moe_decode_grid_override", "moe_decode_wait_test",
    "moe_merge_partial",
    "moe_prefill_create", "moe_prefill_prefetch", "moe_prefill_acquire", "moe_prefill_release",
    "moe_prefill_destroy", "moe_prefill_create_ring", "moe_prefill_finish", "moe_cache_prefill_load",
    "moe_cache_resize",
    "moe_e4m3_to_bf16", "moe_pack_weights", "moe_stream_read", "moe_stream_read_cfg",
    "moe_host_exec_create", "moe_host_exec_destroy", "moe_host_exec_simd", "moe_host_exec_cpus", "moe_host_forward",
    "moe_host_forward_enqueue", "moe_host_exec_status", "moe_host_exec_stats",
    "moe_host_signal", "moe_host_forward_signal", "moe_merge_partial_after", "moe_calibrate_bandwidth",
]


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.moe_last_error().decode(errors="replace")
        super().__init__("%s: %s (%d) %s" % (where, STATUS.get(status, "?"), status, msg))


class Slots(ctypes.Structure):
    _fields_ = [("wtype", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("n_slots", ctypes.c_int32),
                ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


class HostPool(ctypes.Structure):
    _fields_ = [(n, ctypes.POINTER(ctypes.c_void_p)) for n in
                ("w_gate_up", "w_down", "s_gate", "s_up", "s_down")]


class CacheCfg(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("T_max", ctypes.c_int32), ("C", ctypes.c_int32),
                ("bp", ctypes.c_uint32), ("bh", ctypes.c_uint32)]


class StepOutC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("pick_slot", "uniq", "is_hit", "fill_id", "fill_slot", "fill_evicted", "host_id", "counts")]


class Bandwidth(ctypes.Structure):
    _fields_ = [("bp", ctypes.c_uint32), ("bh", ctypes.c_uint32), ("fill_GBps", ctypes.c_double),
                ("dma_GBps", ctypes.c_double), ("host_GBps", ctypes.c_double), ("expert_bytes", ctypes.c_double)]


_vp, _i32, _u32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
_P = ctypes.POINTER
_sig = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_route_topk": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "moe_cache_workspace_bytes": (_i32, [_P(CacheCfg), _P(_sz)]),
    "moe_cache_route_step": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _u32, _P(StepOutC), _vp]),
    "moe_cache_create": (_i32, [_P(CacheCfg), _P(Slots), _P(HostPool), _vp, _sz, _vp, _P(_vp)]),
    "moe_cache_seed": (_i32, [_vp, _P(_i32), _i32, _u32, _vp]),
    "moe_cache_step": (_i32, [_vp, _vp, _vp, _i32, _u32, _P(StepOutC), _vp]),
    "moe_cache_fill": (_i32, [_vp, _P(StepOutC), _vp]),
    "moe_cache_read_state": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_cache_error": (_i32, [_vp, _P(_i32), _vp]),
    "moe_cache_destroy": (_i32, [_vp]),
    "moe_forward_workspace_bytes": (_i32, [_i32, _i32, _i32, _i32, _i32, _u32, _P(_sz)]),
    "moe_expert_forward": (_i32, [_P(Slots), _vp, _vp, _vp, _i32, _i32, _vp, _vp, _sz, _u32, _vp]),
    "moe_expert_forward_merge": (_i32, [_P(Slots), _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz,
                                        _u32, _vp]),
    "moe_expert_forward_merge_static": (_i32, [_P(Slots), _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "moe_decode_grid_override": (_i32, [_i32]),
    "moe_decode_wait_test": (_i32, [_P(Slots), _vp, _vp, _vp, _i32, _i32, _vp, _vp, _sz, _u32, _vp]),
    "moe_merge_partial": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _vp]),
    "moe_stream_read": (_i32, [_vp, _sz, _vp, _vp]),
    "moe_stream_read_cfg": (_i32, [_vp, _sz, _vp, _i32, _i32, _vp]),
    "moe_prefill_create": (_i32, [_vp, _P(_vp)]),
    "moe_prefill_prefetch": (_i32, [_vp, _i32, _vp]),
    "moe_prefill_acquire": (_i32, [_vp, _i32, _vp, _P(Slots)]),
    "moe_prefill_release": (_i32, [_vp, _i32, _vp]),
    "moe_prefill_destroy": (_i32, [_vp, _vp]),
    "moe_prefill_create_ring": (_i32, [_vp, _i32, _P(_vp)]),
    "moe_prefill_finish": (_i32, [_vp, _vp]),
    "moe_cache_prefill_load": (_i32, [_vp, _i32, _vp, _i32, _u32, _P(StepOutC), _vp, _vp]),
    "moe_cache_resize": (_i32, [_vp, _P(Slots), _vp, _sz, _vp]),
    "moe_e4m3_to_bf16": (_i32, [_vp, _vp, ctypes.c_int64, _vp]),
    "moe_pack_weights": (_i32, [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_host_exec_create": (_i32, [_i32, _u32, _P(_vp)]),
    "moe_host_exec_destroy": (_i32, [_vp]),
    "moe_host_exec_simd": (_i32, [_vp]),
    "moe_host_exec_cpus": (_i32, [_vp, _vp, _i32, _P(_i32)]),
    "moe_host_forward": (_i32, [_vp, _P(HostPool), _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _vp]),
    "moe_host_forward_enqueue": (_i32, [_vp, _P(HostPool), _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _vp,
                                        _vp]),
    "moe_host_exec_status": (_i32, [_vp]),
    "moe_host_exec_stats": (_i32, [_vp, _P(ctypes.c_uint64), _P(ctypes.c_uint64)]),
    "moe_host_signal": (_i32, [_vp, _u32, _vp]),
    "moe_host_forward_signal": (_i32, [_vp, _P(HostPool), _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _vp,
                                       _vp, _vp, _u32]),
    "moe_merge_partial_after": (_i32, [_vp, _vp, _vp, _u32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_calibrate_bandwidth": (_i32, [_vp, _vp, _P(_i32), _i32, _P(Slots), _i32, _vp, _P(Bandwidth)]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args


def _check(st, where):
    if st != MOE_OK:
        raise MoeError(st, where)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------- router
def route_topk(logits, k, ids=None, w=None, stream=None):
    """logits float32 [T, E] (cuda) -> (ids int32 [T, k], w float32 [T, k])."""
    assert logits.is_cuda and logits.dtype == torch.float32 and logits.is_contiguous()
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(_lib.moe_route_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream)), "moe_route_topk")
    return ids, w


# ---------------------------------------------------------------- slot pools
class SlotPool:
    """Device banks of n_slots experts (torch tensors, brick format) and their moe_slots view."""

    def __init__(self, n_slots, H, I, wtype=W_BF16, device="cuda"):
        self.n_slots, self.H, self.I, self.wtype = n_slots, H, I, wtype
        dt = torch.uint16 if wtype == W_BF16 else torch.uint8
        self.w_gu = torch.empty((n_slots, 2 * I * H), dtype=dt, device=device)
        self.w_down = torch.empty((n_slots, H * I), dtype=dt, device=device)
        if wtype == W_FP8_B128:
            self.s_gate = torch.empty((n_slots, I // 128, H // 128), dtype=torch.float32, device=device)
            self.s_up = torch.empty((n_slots, I // 128, H // 128), dtype=torch.float32, device=device)
            self.s_down = torch.empty((n_slots, H // 128, I // 128), dtype=torch.float32, device=device)
        else:
            self.s_gate = self.s_up = self.s_down = None
        self.c = Slots(wtype, H, I, n_slots, *[None if t is None else t.data_ptr() for t in
                                                (self.w_gu, self.w_down, self.s_gate, self.s_up, self.s_down)])

    def prefix(self, n):
        """The first n slots of this pool, same memory (an in-place shrink)."""
        v = SlotPool.__new__(SlotPool)
        v.n_slots, v.H, v.I, v.wtype = n, self.H, self.I, self.wtype
        v.w_gu, v.w_down = self.w_gu[:n], self.w_down[:n]
        v.s_gate, v.s_up, v.s_down = [None if t is None else t[:n] for t in (self.s_gate, self.s_up, self.s_down)]
        v.c = Slots(self.wtype, self.H, self.I, n, *[None if t is None else t.data_ptr() for t in
                                                    (v.w_gu, v.w_down, v.s_gate, v.s_up, v.s_down)])
        v.base = getattr(self, "base", self)
        return v

    def banks(self):
        out = [self.w_gu, self.w_down]
        if self.wtype == W_FP8_B128:
            out += [self.s_gate, self.s_up, self.s_down]
        return out


def pack_weights(wtype, w_gate, w_up, w_down, out_gu=None, out_down=None, stream=None):
    """Row-major device weights [n, I, H], [n, I, H], [n, H, I] -> brick banks [n, 2IH], [n, HI]."""
    n, I, H = w_gate.shape
    if out_gu is None:
        out_gu = torch.empty((n, 2 * I * H), dtype=w_gate.dtype, device=w_gate.device)
    if out_down is None:
        out_down = torch.empty((n, H * I), dtype=w_gate.dtype, device=w_gate.device)
    _check(_lib.moe_pack_weights(wtype, H, I, n, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out_gu),
                                 _ptr(out_down), _stream(stream)), "moe_pack_weights")
    return out_gu, out_down


class HostPoolTables:
    """Per-logical-id pointers into pinned host tensors (aliasing allowed).

    `banks` is a list (gate_up, down[, s_gate, s_up, s_down]) of pinned host
    tensors whose first dim indexes *base* experts; `base_of` maps a logical
    id to its base expert row.  pinned=False allows pageable tensors, for the
    host executor alone (fills need pinned memory)."""

    def __init__(self, banks, base_of, n_ids, pinned=True):
        self.banks = banks
        self._arrays = []
        ptrs = []
        for t in banks:
            assert t.is_pinned() or not pinned, "host pool banks must be pinned"
            row = t[0].numel() * t.element_size()
            arr = (ctypes.c_void_p * n_ids)(*[t.data_ptr() + int(base_of(i)) * row for i in range(n_ids)])
            self._arrays.append(arr)
            ptrs.append(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)))
        while len(ptrs) < 5:
            ptrs.append(None)
        self.c = HostPool(*ptrs)


class StepOut:
    """Fixed-shape device outputs of one cache step."""

    def __init__(self, T_max, k, E, device="cuda"):
        self.U_max = min(T_max * k, E)
        mk = lambda n: torch.full((n,), -1, dtype=torch.int32, device=device)
        self.pick_slot = mk(T_max * k)
        self.uniq, self.is_hit = mk(self.U_max), mk(self.U_max)
        self.fill_id, self.fill_slot, self.fill_evicted = mk(self.U_max), mk(self.U_max), mk(self.U_max)
        self.host_id = mk(self.U_max)
        self.counts = torch.zeros((CNT_N,), dtype=torch.int32, device=device)
        self.c = StepOutC(*[t.data_ptr() for t in (self.pick_slot, self.uniq, self.is_hit, self.fill_id,
                                                   self.fill_slot, self.fill_evicted, self.host_id, self.counts)])


class Cache:
    """The shared LRU expert-slot cache (device tables in a torch workspace)."""

    def __init__(self, L, E, k, T_max, slots: SlotPool, host: HostPoolTables, bp, bh, stream=None):
        self.cfg = CacheCfg(L, E, k, T_max, slots.n_slots, bp, bh)
        nbytes = ctypes.c_size_t(0)
        _check(_lib.moe_cache_workspace_bytes(ctypes.byref(self.cfg), ctypes.byref(nbytes)), "workspace_bytes")
        self.ws = torch.empty((nbytes.value,), dtype=torch.uint8, device="cuda")
        self.slots, self.host = slots, host
        h = ctypes.c_void_p()
        _check(_lib.moe_cache_create(ctypes.byref(self.cfg), ctypes.byref(slots.c), ctypes.byref(host.c),
                                     _ptr(self.ws), nbytes.value, _stream(stream), ctypes.byref(h)),
               "moe_cache_create")
        self.h = h
        # device scalars 0 .. L-1: a host layer index is passed as a pointer into this table
        self.layer_tab = torch.arange(L, dtype=torch.int32, device="cuda")

    def _layer_ptr(self, layer):
        """A device int32 scalar holding the layer: a 1-element int32 cuda
        tensor is passed as is, an int through the resident table (an int
        outside [0, L) goes through a fresh scalar, which the kernel rejects)."""
        if isinstance(layer, torch.Tensor):
            assert layer.is_cuda and layer.dtype == torch.int32 and layer.numel() == 1
            return _ptr(layer)
        if 0 <= layer < self.cfg.L:
            return ctypes.c_void_p(self.layer_tab.data_ptr() + 4 * int(layer))
        self._bad_layer = torch.tensor([int(layer)], dtype=torch.int32, device="cuda")
        return _ptr(self._bad_layer)

    def seed(self, ids, copy=True, stream=None):
        arr = (ctypes.c_int32 * max(1, len(ids)))(*[int(i) for i in ids])
        _check(_lib.moe_cache_seed(self.h, arr, len(ids), 0 if copy else STEP_NO_COPY, _stream(stream)),
               "moe_cache_seed")

    def step(self, layer, ids, out: StepOut, copy=True, fill_all=False, stream=None):
        T = ids.shape[0]
        flags = (0 if copy else STEP_NO_COPY) | (STEP_FILL_ALL if fill_all else 0)
        _check(_lib.moe_cache_step(self.h, self._layer_ptr(layer), _ptr(ids), T, flags, ctypes.byref(out.c),
                                   _stream(stream)),
               "moe_cache_step")

    def prefill_load(self, layer, ids, out: StepOut, pick_slot=None, copy=True, stream=None):
        """On-demand loading of a prefill batch (any T): returns pick_slot [T, k]."""
        assert ids.is_cuda and ids.dtype == torch.int32 and ids.is_contiguous()
        if pick_slot is None:
            pick_slot = torch.empty(ids.shape, dtype=torch.int32, device=ids.device)
        _check(_lib.moe_cache_prefill_load(self.h, layer, _ptr(ids), ids.shape[0], 0 if copy else STEP_NO_COPY,
                                           ctypes.byref(out.c), _ptr(pick_slot), _stream(stream)),
               "moe_cache_prefill_load")
        return pick_slot

    def route_step(self, layer, logits, ids, w, out: StepOut, copy=True, stream=None):
        """Router + cache step in one launch; writes ids [T, k] and w [T, k]."""
        T = logits.shape[0]
        assert logits.is_cuda and logits.dtype == torch.float32 and logits.is_contiguous()
        _check(_lib.moe_cache_route_step(self.h, self._layer_ptr(layer), _ptr(logits), T, _ptr(ids), _ptr(w),
                                         0 if copy else STEP_NO_COPY, ctypes.byref(out.c), _stream(stream)),
               "moe_cache_route_step")

    def fill(self, out: StepOut, stream=None):
        _check(_lib.moe_cache_fill(self.h, ctypes.byref(out.c), _stream(stream)), "moe_cache_fill")

    def read_state(self, stream=None):
        import numpy as np
        C, LE = self.cfg.C, self.cfg.L * self.cfg.E
        slot_id = np.empty(C, np.int32)
        stamp = np.empty(C, np.uint64)
        id_slot = np.empty(LE, np.int32)
        tick = np.empty(1, np.uint64)
        counters = np.empty(6, np.uint64)
        _check(_lib.moe_cache_read_state(self.h, slot_id.ctypes.data, stamp.ctypes.data, id_slot.ctypes.data,
                                         tick.ctypes.data, counters.ctypes.data, _stream(stream)), "read_state")
        return slot_id, stamp, id_slot, int(tick[0]), counters

    def error(self, stream=None):
        code = ctypes.c_int32(0)
        _check(_lib.moe_cache_error(self.h, ctypes.byref(code), _stream(stream)), "moe_cache_error")
        return code.value

    def resize(self, slots: SlotPool, stream=None):
        """Safe-point resize to slots.n_slots slots (same memory or new banks)."""
        cfg = CacheCfg(self.cfg.L, self.cfg.E, self.cfg.k, self.cfg.T_max, slots.n_slots, self.cfg.bp, self.cfg.bh)
        nbytes = ctypes.c_size_t(0)
        _check(_lib.moe_cache_workspace_bytes(ctypes.byref(cfg), ctypes.byref(nbytes)), "workspace_bytes")
        ws = torch.empty((nbytes.value,), dtype=torch.uint8, device="cuda")
        _check(_lib.moe_cache_resize(self.h, ctypes.byref(slots.c), _ptr(ws), nbytes.value, _stream(stream)),
               "moe_cache_resize")
        self.cfg, self.ws, self.slots = cfg, ws, slots

    def calibrate(self, ids, scratch: SlotPool, reps=5, host_exec=None, stream=None):
        """moe_calibrate_bandwidth: B_P through the fill kernel (and the DMA
        engines) and B_H through the host executor, on experts `ids` of the
        host pool copied into `scratch`; returns a dict (bp, bh in 0.1 GB/s)."""
        arr = (ctypes.c_int32 * len(ids))(*[int(i) for i in ids])
        r = Bandwidth()
        _check(_lib.moe_calibrate_bandwidth(self.h, host_exec.h if host_exec is not None else None, arr, len(ids),
                                            ctypes.byref(scratch.c), reps, _stream(stream), ctypes.byref(r)),
               "moe_calibrate_bandwidth")
        return {f: getattr(r, f) for f, _ in Bandwidth._fields_}

    def destroy(self):
        if self.h:
            _check(_lib.moe_cache_destroy(self.h), "moe_cache_destroy")
            self.h = None


# ---------------------------------------------------------------- forward / merge
def forward_workspace(T_max, k, H, I, n_slots, mode, device="cuda"):
    n = ctypes.c_size_t(0)
    _check(_lib.moe_forward_workspace_bytes(T_max, k, H, I, n_slots, mode, ctypes.byref(n)),
           "moe_forward_workspace_bytes")
    # zero-filled: decode mode keeps self-resetting counters in it
    return torch.zeros((max(n.value, 256),), dtype=torch.uint8, device=device)


def expert_forward(slots_c, x, pick_slot, w, mode, ws, y=None, stream=None):
    """slots_c: Slots struct; x uint16 [T, H]; pick_slot int32 [T, k]; w float32 [T, k]."""
    T, k = pick_slot.shape
    if y is None:
        y = torch.empty((T, slots_c.H), dtype=torch.float32, device=x.device)
    _check(_lib.moe_expert_forward(ctypes.byref(slots_c), _ptr(x), _ptr(pick_slot), _ptr(w), T, k, _ptr(y),
                                   _ptr(ws), ws.numel(), mode, _stream(stream)), "moe_expert_forward")
    return y


def expert_forward_merge(slots_c, x, pick_slot, w, mode, ws, y_host, y_out=None, y_gpu=None, y_out_bf16=None,
                         stream=None):
    """expert_forward then merge_partial in one call: y_out = y_gpu + y_host
    (y_gpu, the GPU partial sum, is written only when given)."""
    T, k = pick_slot.shape
    if y_out is None:
        y_out = torch.empty((T, slots_c.H), dtype=torch.float32, device=x.device)
    _check(_lib.moe_expert_forward_merge(ctypes.byref(slots_c), _ptr(x), _ptr(pick_slot), _ptr(w), T, k,
                                         _ptr(y_gpu), _ptr(y_host), _ptr(y_out), _ptr(y_out_bf16),
                                         _ptr(ws), ws.numel(), mode, _stream(stream)), "moe_expert_forward_merge")
    return y_out


def expert_forward_merge_static(slots_c, x, pick_slot, w, y_host, y_out=None, y_gpu=None, y_out_bf16=None,
                                stream=None):
    """expert_forward_merge in decode mode with the library's static device
    scratch as its workspace (no allocation by the library)."""
    T, k = pick_slot.shape
    if y_out is None:
        y_out = torch.empty((T, slots_c.H), dtype=torch.float32, device=x.device)
    _check(_lib.moe_expert_forward_merge_static(ctypes.byref(slots_c), _ptr(x), _ptr(pick_slot), _ptr(w), T, k,
                                                _ptr(y_gpu), _ptr(y_host), _ptr(y_out), _ptr(y_out_bf16),
                                                _stream(stream)), "moe_expert_forward_merge_static")
    return y_out


def decode_grid_override(n_workgroups):
    """Fix the decode forward's grid to n_workgroups for later launches in this
    process (0: automatic)."""
    _check(_lib.moe_decode_grid_override(int(n_workgroups)), "moe_decode_grid_override")


def decode_wait_test(slots_c, x, pick_slot, w, ws, polls, y=None, stream=None):
    """The down phase of the decode forward alone, with the one-launch form's
    bounded waits and at most `polls` polls: every waiting workgroup gives up
    and sets ws's first word (y is then not valid)."""
    T, k = pick_slot.shape
    if y is None:
        y = torch.empty((T, slots_c.H), dtype=torch.float32, device=x.device)
    _check(_lib.moe_decode_wait_test(ctypes.byref(slots_c), _ptr(x), _ptr(pick_slot), _ptr(w), T, k, _ptr(y),
                                     _ptr(ws), ws.numel(), int(polls), _stream(stream)), "moe_decode_wait_test")
    return y


def merge_partial(y_gpu, y_host, y_out=None, y_out_bf16=None, stream=None):
    T, H = y_gpu.shape
    if y_out is None:
        y_out = torch.empty_like(y_gpu)
    _check(_lib.moe_merge_partial(_ptr(y_gpu), _ptr(y_host), T, H, _ptr(y_out), _ptr(y_out_bf16),
                                  _stream(stream)), "moe_merge_partial")
    return y_out


def host_signal(word, seq, stream=None):
    """In stream order, store seq into the pinned uint32 word."""
    _check(_lib.moe_host_signal(_ptr(word), seq & 0xFFFFFFFF, _stream(stream)), "moe_host_signal")


def merge_partial_after(y_gpu, y_host, done, seq, y_out=None, y_out_bf16=None, err=None, stream=None):
    """moe_merge_partial after waiting (bounded) for done >= seq."""
    T, H = y_gpu.shape
    if y_out is None:
        y_out = torch.empty_like(y_gpu)
    _check(_lib.moe_merge_partial_after(_ptr(y_gpu), _ptr(y_host), _ptr(done), seq & 0xFFFFFFFF, T, H, _ptr(y_out),
                                        _ptr(y_out_bf16), _ptr(err), _stream(stream)), "moe_merge_partial_after")
    return y_out


def stream_read(src, sink, stream=None):
    """One launch that only reads src (a measurement reference)."""
    _check(_lib.moe_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)),
           "moe_stream_read")


def stream_read_cfg(src, sink, n_wg, unroll, stream=None):
    """moe_stream_read with n_wg workgroups and `unroll` loads in flight per thread."""
    _check(_lib.moe_stream_read_cfg(_ptr(src), src.numel() * src.element_size(), _ptr(sink), n_wg, unroll,
                                    _stream(stream)), "moe_stream_read_cfg")


def e4m3_to_bf16(codes, out=None, stream=None):
    """Exact expansion of E4M3FN codes (uint8, cuda) to BF16 bits with the kernels' routine."""
    if out is None:
        out = torch.empty(codes.shape, dtype=torch.uint16, device=codes.device)
    _check(_lib.moe_e4m3_to_bf16(_ptr(codes), _ptr(out), codes.numel(), _stream(stream)), "moe_e4m3_to_bf16")
    return out


# ---------------------------------------------------------------- prefill double buffer
class PrefillPool:
    """depth full-layer buffers (2: the double buffer) reserved from the cache's slots."""

    def __init__(self, cache: Cache, depth=2):
        h = ctypes.c_void_p()
        if depth == 2:
            _check(_lib.moe_prefill_create(cache.h, ctypes.byref(h)), "moe_prefill_create")
        else:
            _check(_lib.moe_prefill_create_ring(cache.h, depth, ctypes.byref(h)), "moe_prefill_create_ring")
        self.h, self.cache, self.depth = h, cache, depth

    def prefetch(self, layer, copy_stream):
        _check(_lib.moe_prefill_prefetch(self.h, layer, _stream(copy_stream)), "moe_prefill_prefetch")

    def acquire(self, layer, compute=None):
        v = Slots()
        _check(_lib.moe_prefill_acquire(self.h, layer, _stream(compute), ctypes.byref(v)), "moe_prefill_acquire")
        return v

    def release(self, layer, compute=None):
        _check(_lib.moe_prefill_release(self.h, layer, _stream(compute)), "moe_prefill_release")

    def destroy(self, stream=None):
        """End prefill discarding the buffers (their slots return empty)."""
        if self.h:
            _check(_lib.moe_prefill_destroy(self.h, _stream(stream)), "moe_prefill_destroy")
            self.h = None

    def finish(self, stream=None):
        """End prefill keeping what the buffers hold as decode's residents."""
        if self.h:
            _check(_lib.moe_prefill_finish(self.h, _stream(stream)), "moe_prefill_finish")
            self.h = None


# ---------------------------------------------------------------- host executor
class HostExec:
    """The CPU executor of the host set (moe_host_forward): a persistent pool
    of n_threads threads (the caller counts as one)."""

    def __init__(self, n_threads, portable=False, pin=False):
        h = ctypes.c_void_p()
        flags = (HOST_PORTABLE if portable else 0) | (HOST_PIN if pin else 0)
        _check(_lib.moe_host_exec_create(n_threads, flags, ctypes.byref(h)), "moe_host_exec_create")
        self.h = h
        self.n_threads = n_threads

    def simd(self):
        return _lib.moe_host_exec_simd(self.h)

    def cpus(self):
        """(CPU of each thread, -1 where not pinned; the GPU's NUMA node or -1)."""
        arr = (ctypes.c_int32 * self.n_threads)()
        node = ctypes.c_int32(-1)
        _check(_lib.moe_host_exec_cpus(self.h, arr, self.n_threads, ctypes.byref(node)), "moe_host_exec_cpus")
        return list(arr), node.value

    def forward(self, pool, wtype, H, I, x, ids, pick_slot, w, y_host=None):
        """Host tensors: x uint16 [T, H] (BF16 bits), ids / pick_slot int32
        [T, k], w float32 [T, k]; returns y_host float32 [T, H] (host)."""
        T, k = ids.shape
        for t in (x, ids, pick_slot, w):
            assert not t.is_cuda and t.is_contiguous()
        if y_host is None:
            y_host = torch.empty((T, H), dtype=torch.float32)
        _check(_lib.moe_host_forward(self.h, ctypes.byref(pool.c), wtype, H, I, _ptr(x), _ptr(ids), _ptr(pick_slot),
                                     _ptr(w), T, k, _ptr(y_host)), "moe_host_forward")
        return y_host

    def enqueue(self, pool, wtype, H, I, x, ids, pick_slot, w, y_host, stream=None):
        """Stream-ordered forward: host tensors (pinned where the GPU copies
        into or reads them) that must stay alive until the stream passes."""
        T, k = ids.shape
        for t in (x, ids, pick_slot, w, y_host):
            assert not t.is_cuda and t.is_contiguous()
        self._keep = (pool, x, ids, pick_slot, w, y_host)
        _check(_lib.moe_host_forward_enqueue(self.h, ctypes.byref(pool.c), wtype, H, I, _ptr(x), _ptr(ids),
                                             _ptr(pick_slot), _ptr(w), T, k, _ptr(y_host), _stream(stream)),
               "moe_host_forward_enqueue")

    def forward_signal(self, pool, wtype, H, I, x, ids, pick_slot, w, y_host, ready, done, seq):
        """Queue a call on the dispatcher thread: it waits for ready >= seq,
        computes y_host, then stores seq into done (pinned uint32 words)."""
        T, k = ids.shape
        for t in (x, ids, pick_slot, w, y_host, ready, done):
            assert not t.is_cuda and t.is_contiguous()
        self._keep_sig = (pool, x, ids, pick_slot, w, y_host, ready, done)
        _check(_lib.moe_host_forward_signal(self.h, ctypes.byref(pool.c), wtype, H, I, _ptr(x), _ptr(ids),
                                            _ptr(pick_slot), _ptr(w), T, k, _ptr(y_host), _ptr(ready), _ptr(done),
                                            seq & 0xFFFFFFFF), "moe_host_forward_signal")

    def status(self):
        """First failure of an enqueued run since the last call (0 if none)."""
        return _lib.moe_host_exec_status(self.h)

    def stats(self):
        """(calls with host picks, seconds spent in them) since creation."""
        c, ns = ctypes.c_uint64(0), ctypes.c_uint64(0)
        _check(_lib.moe_host_exec_stats(self.h, ctypes.byref(c), ctypes.byref(ns)), "moe_host_exec_stats")
        return c.value, ns.value / 1e9

    def destroy(self):
        if self.h:
            _check(_lib.moe_host_exec_destroy(self.h), "moe_host_exec_destroy")
            self.h = None
