"""Python binding of libdita: selective attention-state reuse on MI355X.

Argument marshalling only.  Every step of the hot path runs in the HIP
library (``libdita.so``, built in-tree by ``partial_state_reuse_amd.build``);
PyTorch only supplies device memory and the current stream.  Importing this
package fails loudly when the library has not been built: there is no
fallback of any kind.

The functions carry the names of the C entry points declared in
``include/dita.h``:

    dita_attn_partial   fresh attention state (O_p, LSE_p) of Q against one K/V partition
    dita_state_merge    exact LSE-weighted merge of P states
    dita_state_cache_*  device-resident per-partition state store (``StateCache`` wraps them)
    dita_plan_mask      host reuse-mask planner
    dita_attn_step      one compute-or-reuse rank-step over all P partitions
    dita_attn_step_ex   the same, with reused states pre-merged on a side stream
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdita.so")

DITA_OK, DITA_ERR_ARG, DITA_ERR_SHAPE, DITA_ERR_DTYPE = 0, 1, 2, 3
DITA_ERR_STATE, DITA_ERR_ALIGN, DITA_ERR_HIP, DITA_ERR_SIZE = 4, 5, 6, 7
DITA_F32, DITA_BF16 = 0, 1
DITA_PLAN_DIST, DITA_PLAN_KNEAREST, DITA_PLAN_RANDOM, DITA_PLAN_RAMP = 0, 1, 2, 3
DITA_STATE_NONE, DITA_STATE_FULL, DITA_STATE_COMPACT, DITA_STATE_HOST = 0, 1, 2, 3
MAX_PARTITIONS = 64


class DitaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {_lib.dita_status_str(status).decode()} (status {status})"
        if status == DITA_ERR_HIP:
            msg += f", hipError {_lib.dita_last_hip_error()}"
        super().__init__(msg)


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("Nq", ctypes.c_int64), ("scale", ctypes.c_float)]


class Plan(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int32), ("q", ctypes.c_int32), ("policy", ctypes.c_int32),
                ("radius", ctypes.c_int32), ("radius_end", ctypes.c_int32),
                ("k_nearest", ctypes.c_int32), ("anchor_period", ctypes.c_int32),
                ("total_steps", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class StepInfo(ctypes.Structure):
    _fields_ = [("n_fresh", ctypes.c_int32), ("n_reused", ctypes.c_int32),
                ("fresh_flops", ctypes.c_double), ("merge_bytes", ctypes.c_double),
                ("ev_begin", ctypes.c_void_p), ("ev_attn_end", ctypes.c_void_p),
                ("ev_end", ctypes.c_void_p), ("merge_sources", ctypes.c_int32),
                ("premerge_sources", ctypes.c_int32), ("premerge_bytes", ctypes.c_double),
                ("fetched", ctypes.c_int32), ("composed", ctypes.c_int32)]


class ErrorPlan(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int32), ("q", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("anchor_period", ctypes.c_int32), ("budget", ctypes.c_double),
                ("fresh_weight", ctypes.c_double)]


class AttnLayout(ctypes.Structure):
    _fields_ = [("big_tiles", ctypes.c_int32), ("small_tiles", ctypes.c_int32),
                ("dual_tails", ctypes.c_int32), ("workgroups", ctypes.c_int64), ("split_units", ctypes.c_int32),
                ("split_tiles", ctypes.c_int32), ("max_pieces", ctypes.c_int32),
                ("compute_units", ctypes.c_int32), ("scratch_bytes", ctypes.c_int64),
                ("scratch_allocated", ctypes.c_int64), ("staged_pairs", ctypes.c_int32),
                ("small_tiles_b", ctypes.c_int32)]


class StepOpts(ctypes.Structure):
    _fields_ = [("side_stream", ctypes.c_void_p), ("min_premerge", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("compose_next", ctypes.POINTER(ctypes.c_uint8))]


def _load() -> ctypes.CDLL:
    # torch must bring in its HIP runtime first: libdita then binds to that same runtime
    # (both carry the soname libamdhip64.so.7).  Loaded the other way round, torch would
    # load a second HIP runtime into the process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python partial_state_reuse_amd/build.py` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    pvp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "dita_status_str": (ctypes.c_char_p, [i32]),
        "dita_last_hip_error": (i32, []),
        "dita_version": (i32, []),
        "dita_attn_partial": (i32, [ctypes.POINTER(Shape), vp, vp, vp, i64, vp, vp, vp]),
        "dita_attn_launch_info": (i32, [ctypes.POINTER(Shape), i32, i64, ctypes.POINTER(AttnLayout)]),
        "dita_state_merge": (i32, [ctypes.POINTER(Shape), i32, pvp, pvp, vp, vp, vp]),
        "dita_state_cache_bytes": (sz, [ctypes.POINTER(Shape), i32]),
        "dita_state_cache_init": (i32, [pvp, ctypes.POINTER(Shape), i32, vp, sz]),
        "dita_state_cache_init_pool": (i32, [pvp, ctypes.POINTER(Shape), i32, i32, vp, sz]),
        "dita_state_cache_bytes_compact": (sz, [ctypes.POINTER(Shape), i32, i32]),
        "dita_state_cache_init_compact": (i32, [pvp, ctypes.POINTER(Shape), i32, i32, i32, vp, sz]),
        "dita_state_cache_compact": (i32, [vp, i32, vp]),
        "dita_state_cache_compact_slot": (i32, [vp, i32, pvp, pvp, pvp]),
        "dita_state_cache_format": (i32, [vp, i32, ctypes.POINTER(ctypes.c_int)]),
        "dita_state_cache_offload": (i32, [vp, i32, vp, vp, vp]),
        "dita_state_cache_fetch": (i32, [vp, i32, vp]),
        "dita_state_cache_residency": (i32, [vp, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                             ctypes.POINTER(ctypes.c_int)]),
        "dita_state_cache_free": (i32, [vp]),
        "dita_state_cache_slot": (i32, [vp, i32, pvp, pvp]),
        "dita_state_cache_store": (i32, [vp, i32, vp, vp, i64, vp]),
        "dita_state_cache_load": (i32, [vp, i32, vp, vp, vp]),
        "dita_state_cache_invalidate": (i32, [vp, i32]),
        "dita_state_cache_info": (i32, [vp, i32, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(i64)]),
        "dita_state_cache_shape": (i32, [vp, ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_int)]),
        "dita_plan_mask": (i32, [ctypes.POINTER(Plan), vp, i64, ctypes.POINTER(ctypes.c_uint8)]),
        "dita_plan_bits": (i32, [ctypes.POINTER(Plan), vp, i64, ctypes.POINTER(ctypes.c_uint64)]),
        "dita_mask_to_bits": (i32, [ctypes.POINTER(ctypes.c_uint8), i32, ctypes.POINTER(ctypes.c_uint64)]),
        "dita_mask_from_bits": (i32, [ctypes.c_uint64, i32, ctypes.POINTER(ctypes.c_uint8)]),
        "dita_state_cache_compose": (i32, [vp, i32, i32, vp]),
        "dita_state_cache_compose_runs": (i32, [vp, ctypes.POINTER(ctypes.c_uint8), vp,
                                                ctypes.POINTER(ctypes.c_int)]),
        "dita_state_cache_group": (i32, [vp, i32, ctypes.POINTER(ctypes.c_int),
                                         ctypes.POINTER(ctypes.c_int)]),
        "dita_state_cache_live": (i32, [vp, ctypes.POINTER(ctypes.c_int)]),
        "dita_state_cache_effective_mask": (i32, [vp, ctypes.POINTER(ctypes.c_uint8),
                                                  ctypes.POINTER(ctypes.c_uint8)]),
        "dita_attn_step": (i32, [vp, vp, pvp, pvp, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_uint8),
                                 i64, vp, vp, vp, ctypes.POINTER(StepInfo)]),
        "dita_attn_step_ex": (i32, [vp, vp, pvp, pvp, ctypes.POINTER(i64),
                                    ctypes.POINTER(ctypes.c_uint8), i64, vp, vp, vp,
                                    ctypes.POINTER(StepOpts), ctypes.POINTER(StepInfo)]),
        "dita_state_contrib": (i32, [ctypes.POINTER(Shape), i32, pvp, vp, vp, vp]),
        "dita_state_cache_contrib": (i32, [vp, vp, vp, vp]),
        "dita_state_change": (i32, [ctypes.POINTER(Shape), vp, vp, vp, vp, i32, vp, vp]),
        "dita_state_change_noalloc": (i32, [ctypes.POINTER(Shape), vp, vp, vp, vp, i32, vp, vp]),
        "dita_planner_create": (i32, [pvp, ctypes.POINTER(ErrorPlan)]),
        "dita_planner_free": (i32, [vp]),
        "dita_planner_set_weights": (i32, [vp, ctypes.POINTER(ctypes.c_double)]),
        "dita_planner_observe": (i32, [vp, i64, ctypes.c_double]),
        "dita_planner_mask": (i32, [vp, i64, ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(i64),
                                    ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_double)]),
        "dita_planner_mask_cache": (i32, [vp, vp, i64, ctypes.POINTER(ctypes.c_uint8),
                                          ctypes.POINTER(ctypes.c_double)]),
        "dita_event_create": (i32, [pvp]),
        "dita_event_destroy": (i32, [vp]),
        "dita_event_record": (i32, [vp, vp]),
        "dita_event_elapsed_ms": (i32, [vp, vp, ctypes.POINTER(ctypes.c_float)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    """The loaded shared library (for symbol checks and raw calls)."""
    return _lib


def _check(status: int, where: str) -> None:
    if status != DITA_OK:
        raise DitaError(status, where)


# --------------------------------------------------------------------------- marshalling


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DITA_BF16
    if t.dtype == torch.float32:
        return DITA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(t, stream=None) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream


def _expect(t, shape, dtype, name: str):
    """Raise ValueError unless ``t`` has exactly ``shape`` and ``dtype`` (checked before
    any pointer is taken: the C ABI cannot see buffer sizes)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _same_device(name: str, ref, *ts):
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name}: tensors on {t.device} and {ref.device}")


def _check_kv(k, v, B: int, H: int, D: int, dtype, name: str):
    if k.dim() != 4 or tuple(k.shape[:2]) != (B, H) or k.shape[3] != D or k.shape[2] < 1:
        raise ValueError(f"{name}: K has shape {tuple(k.shape)}, expected [{B}, {H}, Nk >= 1, {D}]")
    _expect(k, k.shape, dtype, f"{name} K")
    _expect(v, k.shape, dtype, f"{name} V")


def make_shape(q, scale: float = 0.0) -> Shape:
    """Shape record of a [B, H, Nq, D] query tensor."""
    B, H, Nq, D = q.shape
    return Shape(B, H, D, _dtype_code(q), Nq, float(scale))


def _ptr_array(ptrs: Sequence[Optional[int]]):
    arr = (ctypes.c_void_p * len(ptrs))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


# --------------------------------------------------------------------------- entry points


def dita_attn_partial(q, k, v, o=None, lse=None, scale: float = 0.0, stream=None):
    """Fresh state (O_p, LSE_p) of ``q`` [B,H,Nq,D] against one partition ``k``, ``v`` [B,H,Nk,D]."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, Nq, D], got shape {tuple(q.shape)}")
    B, H, Nq, D = q.shape
    _check_kv(k, v, B, H, D, q.dtype, "dita_attn_partial")
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _expect(o, q.shape, q.dtype, "o")
    _expect(lse, (B, H, Nq), torch.float32, "lse")
    _same_device("dita_attn_partial", q, k, v, o, lse)
    shape = make_shape(q, scale)
    _check(_lib.dita_attn_partial(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), k.shape[2],
                                  _ptr(o), _ptr(lse), _stream(q, stream)), "dita_attn_partial")
    return o, lse


def dita_attn_launch_info(B: int, H: int, Nq: int, D: int, n_blocks: int = 1, nk: int = 0) -> dict:
    """Work layout of the bf16 attention kernel on the current device for ``n_blocks``
    fresh blocks of ``nk`` keys each (``nk`` <= 0: unequal lengths); see AttnLayout."""
    out = AttnLayout()
    shape = Shape(B, H, D, DITA_BF16, Nq, 0.0)
    _check(_lib.dita_attn_launch_info(ctypes.byref(shape), n_blocks, nk, ctypes.byref(out)),
           "dita_attn_launch_info")
    return {name: getattr(out, name) for name, _ in AttnLayout._fields_}


def dita_state_merge(o_list: Sequence, lse_list: Sequence, o=None, lse=None, scale: float = 0.0,
                     stream=None):
    """Merge P states (lists of [B,H,Nq,D] outputs and [B,H,Nq] fp32 LSEs)."""
    torch = _torch()
    if len(o_list) != len(lse_list) or not o_list:
        raise ValueError("need equally long, non-empty state lists")
    ref = o_list[0]
    if ref.dim() != 4:
        raise ValueError(f"state outputs must be [B, H, Nq, D], got shape {tuple(ref.shape)}")
    for x in o_list:
        if x.shape != ref.shape or x.dtype != ref.dtype:
            raise ValueError("state outputs must share shape and dtype")
    for x in lse_list:
        if x.shape != ref.shape[:3] or x.dtype != torch.float32:
            raise ValueError("LSE arrays must be float32 [B, H, Nq]")
    if o is None:
        o = torch.empty_like(ref)
    if lse is None:
        lse = torch.empty(ref.shape[:3], dtype=torch.float32, device=ref.device)
    _expect(o, ref.shape, ref.dtype, "o")
    _expect(lse, ref.shape[:3], torch.float32, "lse")
    _same_device("dita_state_merge", ref, *o_list, *lse_list, o, lse)
    shape = make_shape(ref, scale)
    P = len(o_list)
    _check(_lib.dita_state_merge(ctypes.byref(shape), P, _ptr_array([_ptr(x) for x in o_list]),
                                 _ptr_array([_ptr(x) for x in lse_list]), _ptr(o), _ptr(lse),
                                 _stream(ref, stream)), "dita_state_merge")
    return o, lse


def dita_plan_mask(plan: Plan, step: int, cache: Optional["StateCache"] = None) -> np.ndarray:
    """Host reuse mask (uint8[P], 1 = reuse) from the library's planner."""
    out = (ctypes.c_uint8 * plan.P)()
    _check(_lib.dita_plan_mask(ctypes.byref(plan), cache.handle if cache else None, step, out),
           "dita_plan_mask")
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def dita_plan_bits(plan: Plan, step: int, cache: Optional["StateCache"] = None) -> int:
    """The planner's mask as a 64-bit word (bit p set = reuse partition p)."""
    out = ctypes.c_uint64()
    _check(_lib.dita_plan_bits(ctypes.byref(plan), cache.handle if cache else None, step,
                               ctypes.byref(out)), "dita_plan_bits")
    return out.value


class StateCache:
    """Device-resident (O_p, LSE_p) slots (the dita_state_cache_* calls).

    The device buffer is a torch uint8 tensor owned by this object; the C
    handle only records its address.  ``slots`` < P makes a pooled cache of that
    many physical slots (dita_state_cache_init_pool).  Host buffers of offloaded
    states are pinned tensors kept alive here until the state comes back.
    """

    def __init__(self, B: int, H: int, Nq: int, D: int, dtype, P: int, device="cuda",
                 scale: float = 0.0, slots: Optional[int] = None, compact_slots: int = 0):
        torch = _torch()
        code = DITA_BF16 if dtype == torch.bfloat16 else DITA_F32 if dtype == torch.float32 else None
        if code is None:
            raise TypeError(f"unsupported dtype {dtype}")
        self.shape = Shape(B, H, D, code, Nq, float(scale))
        self.P = P
        self.dtype = dtype
        self.slots = P if slots is None else int(slots)
        self.compact_slots = int(compact_slots)
        pooled = slots is not None or self.compact_slots > 0
        if self.compact_slots > 0:
            nbytes = _lib.dita_state_cache_bytes_compact(ctypes.byref(self.shape), self.slots,
                                                         self.compact_slots)
        else:
            nbytes = _lib.dita_state_cache_bytes(ctypes.byref(self.shape), self.slots)
        if nbytes == 0:
            raise ValueError("invalid cache shape or slot count")
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        if self.compact_slots > 0:
            _check(_lib.dita_state_cache_init_compact(ctypes.byref(h), ctypes.byref(self.shape), P,
                                                      self.slots, self.compact_slots,
                                                      self.buffer.data_ptr(), nbytes),
                   "dita_state_cache_init_compact")
        elif pooled:
            _check(_lib.dita_state_cache_init_pool(ctypes.byref(h), ctypes.byref(self.shape), P,
                                                   self.slots, self.buffer.data_ptr(), nbytes),
                   "dita_state_cache_init_pool")
        else:
            _check(_lib.dita_state_cache_init(ctypes.byref(h), ctypes.byref(self.shape), P,
                                              self.buffer.data_ptr(), nbytes), "dita_state_cache_init")
        self.handle = h.value
        self._host = {}
        # partition p owns slot p unless the cache is pooled: the views never change
        self._views = None if pooled else [self._slot_views(p) for p in range(P)]

    def _slot_views(self, p: int):
        torch = _torch()
        o_ptr, l_ptr = ctypes.c_void_p(), ctypes.c_void_p()
        _check(_lib.dita_state_cache_slot(self.handle, p, ctypes.byref(o_ptr), ctypes.byref(l_ptr)),
               "dita_state_cache_slot")
        s = self.shape
        base = self.buffer.data_ptr()
        esz = 2 if s.dtype == DITA_BF16 else 4
        n = s.B * s.H * s.Nq
        o = self.buffer[o_ptr.value - base: o_ptr.value - base + n * s.D * esz]
        lse = self.buffer[l_ptr.value - base: l_ptr.value - base + n * 4]
        return (o.view(self.dtype).view(s.B, s.H, s.Nq, s.D),
                lse.view(torch.float32).view(s.B, s.H, s.Nq))

    def state_shape(self):
        s = self.shape
        return (s.B, s.H, s.Nq, s.D), (s.B, s.H, s.Nq)

    def _check_state(self, o, lse, what: str):
        torch = _torch()
        so, sl = self.state_shape()
        _expect(o, so, self.dtype, f"{what} O")
        _expect(lse, sl, torch.float32, f"{what} LSE")
        _same_device(what, self.buffer, o, lse)

    def slot(self, p: int):
        """Views (O_p, LSE_p) of the device memory of partition p's slot."""
        return self._views[p] if self._views is not None else self._slot_views(p)

    def compact(self, p: int, stream=None):
        """Encode leader p's full state into a compact slot (int8 codes, per-row scale)."""
        _check(_lib.dita_state_cache_compact(self.handle, p, _stream(self.buffer, stream)),
               "dita_state_cache_compact")

    def compact_slot(self, p: int):
        """Views (codes int8 [B,H,Nq,D], scale float32 [B,H,Nq], LSE float32 [B,H,Nq]) of
        p's compact state."""
        torch = _torch()
        c, sc, l = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        _check(_lib.dita_state_cache_compact_slot(self.handle, p, ctypes.byref(c), ctypes.byref(sc),
                                                  ctypes.byref(l)), "dita_state_cache_compact_slot")
        s = self.shape
        base = self.buffer.data_ptr()
        n = s.B * s.H * s.Nq

        def view(ptr, nbytes):
            return self.buffer[ptr - base: ptr - base + nbytes]
        return (view(c.value, n * s.D).view(torch.int8).view(s.B, s.H, s.Nq, s.D),
                view(sc.value, n * 4).view(torch.float32).view(s.B, s.H, s.Nq),
                view(l.value, n * 4).view(torch.float32).view(s.B, s.H, s.Nq))

    def format(self, p: int) -> int:
        """DITA_STATE_NONE, _FULL, _COMPACT or _HOST for partition p's own state."""
        f = ctypes.c_int()
        _check(_lib.dita_state_cache_format(self.handle, p, ctypes.byref(f)), "dita_state_cache_format")
        return f.value

    def offload(self, p: int, stream=None):
        """Move leader p's state to pinned host memory (copies on ``stream``)."""
        torch = _torch()
        s = self.shape
        ho = torch.empty((s.B, s.H, s.Nq, s.D), dtype=self.dtype, pin_memory=True)
        hl = torch.empty((s.B, s.H, s.Nq), dtype=torch.float32, pin_memory=True)
        _check(_lib.dita_state_cache_offload(self.handle, p, ho.data_ptr(), hl.data_ptr(),
                                             _stream(self.buffer, stream)), "dita_state_cache_offload")
        self._host[p] = (ho, hl)
        return ho, hl

    def fetch(self, p: int, stream=None):
        _check(_lib.dita_state_cache_fetch(self.handle, p, _stream(self.buffer, stream)),
               "dita_state_cache_fetch")

    def residency(self):
        """(states on the device, states on the host, free physical slots)."""
        a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check(_lib.dita_state_cache_residency(self.handle, ctypes.byref(a), ctypes.byref(b),
                                               ctypes.byref(c)), "dita_state_cache_residency")
        return a.value, b.value, c.value

    def store(self, p: int, o, lse, step: int, stream=None):
        self._check_state(o, lse, "StateCache.store")
        _check(_lib.dita_state_cache_store(self.handle, p, _ptr(o), _ptr(lse), step,
                                           _stream(o, stream)), "dita_state_cache_store")

    def load(self, p: int, o=None, lse=None, stream=None):
        torch = _torch()
        s = self.shape
        if o is None:
            o = torch.empty((s.B, s.H, s.Nq, s.D), dtype=self.dtype, device=self.buffer.device)
        if lse is None:
            lse = torch.empty((s.B, s.H, s.Nq), dtype=torch.float32, device=self.buffer.device)
        self._check_state(o, lse, "StateCache.load")
        _check(_lib.dita_state_cache_load(self.handle, p, _ptr(o), _ptr(lse), _stream(o, stream)),
               "dita_state_cache_load")
        return o, lse

    def invalidate(self, p: int = -1):
        _check(_lib.dita_state_cache_invalidate(self.handle, p), "dita_state_cache_invalidate")

    def info(self, p: int):
        valid, stamp = ctypes.c_int(), ctypes.c_int64()
        _check(_lib.dita_state_cache_info(self.handle, p, ctypes.byref(valid), ctypes.byref(stamp)),
               "dita_state_cache_info")
        return bool(valid.value), stamp.value

    def valid_mask(self) -> np.ndarray:
        return np.array([self.info(p)[0] for p in range(self.P)], dtype=np.uint8)

    def compose(self, first: int, last: int, stream=None):
        """Merge the states of partitions first..last into one group state in slot ``first``."""
        st = _stream(self.buffer, stream)
        _check(_lib.dita_state_cache_compose(self.handle, first, last, st), "dita_state_cache_compose")

    def compose_runs(self, reuse_mask, stream=None) -> int:
        """Compose every run of partitions ``reuse_mask`` marks for reuse; returns the
        number of merge launches."""
        mask = np.ascontiguousarray(np.asarray(reuse_mask, dtype=np.uint8))
        if mask.shape != (self.P,):
            raise ValueError("reuse mask must have P entries")
        m = (ctypes.c_uint8 * self.P).from_buffer_copy(mask.tobytes())
        n = ctypes.c_int()
        _check(_lib.dita_state_cache_compose_runs(self.handle, m, _stream(self.buffer, stream),
                                                  ctypes.byref(n)), "dita_state_cache_compose_runs")
        return n.value

    def contrib(self, lse, w=None, stream=None):
        """Device float64 [P]: each slot's share exp(LSE_p - lse) averaged over rows."""
        torch = _torch()
        if w is None:
            w = torch.empty(self.P, dtype=torch.float64, device=self.buffer.device)
        _expect(lse, self.state_shape()[1], torch.float32, "StateCache.contrib LSE")
        _expect(w, (self.P,), torch.float64, "StateCache.contrib w")
        _same_device("StateCache.contrib", self.buffer, lse, w)
        _check(_lib.dita_state_cache_contrib(self.handle, _ptr(lse), _ptr(w), _stream(lse, stream)),
               "dita_state_cache_contrib")
        return w

    def group(self, p: int):
        """(first, last) of the group holding partition p."""
        a, b = ctypes.c_int(), ctypes.c_int()
        _check(_lib.dita_state_cache_group(self.handle, p, ctypes.byref(a), ctypes.byref(b)),
               "dita_state_cache_group")
        return a.value, b.value

    def leaders(self) -> List[int]:
        return [p for p in range(self.P) if self.group(p)[0] == p]

    def live(self) -> int:
        n = ctypes.c_int()
        _check(_lib.dita_state_cache_live(self.handle, ctypes.byref(n)), "dita_state_cache_live")
        return n.value

    def effective_mask(self, reuse_mask) -> np.ndarray:
        """The mask a step applies for ``reuse_mask`` (groups are reused or recomputed whole)."""
        mask = np.ascontiguousarray(np.asarray(reuse_mask, dtype=np.uint8))
        if mask.shape != (self.P,):
            raise ValueError("reuse mask must have P entries")
        m = (ctypes.c_uint8 * self.P).from_buffer_copy(mask.tobytes())
        out = (ctypes.c_uint8 * self.P)()
        _check(_lib.dita_state_cache_effective_mask(self.handle, m, out),
               "dita_state_cache_effective_mask")
        return np.frombuffer(bytes(out), dtype=np.uint8).copy()

    def close(self):
        if self.handle:
            _lib.dita_state_cache_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dita_attn_step(cache: StateCache, q, k_list: Sequence, v_list: Sequence, reuse_mask,
                   step: int, o=None, lse=None, stream=None, events=None, side_stream=None,
                   min_premerge: int = 0, compose_next=None) -> StepInfo:
    """One rank-step: fresh states into their slots, reused slots kept, all groups merged.

    ``k_list``/``v_list`` hold P tensors [B,H,Nk_p,D] (entries of reused partitions may
    be None).  ``events``: optional (begin, attn_end, end) raw hipEvent_t handles.
    ``side_stream`` (a torch stream) and ``compose_next`` (the next step's reuse mask:
    its runs are composed into groups by the step, the largest by the final merge
    itself) select ``dita_attn_step_ex``; on the side stream reused states are
    pre-merged while the fresh attention runs.  Returns (o, lse, StepInfo).
    """
    torch = _torch()
    P = cache.P
    if len(k_list) != P or len(v_list) != P:
        raise ValueError("need P key and value tensors")
    mask = np.ascontiguousarray(np.asarray(reuse_mask, dtype=np.uint8))
    if mask.shape != (P,):
        raise ValueError("reuse mask must have P entries")
    s = cache.shape
    so, sl = cache.state_shape()
    _expect(q, so, cache.dtype, "q")
    for p, (k, v) in enumerate(zip(k_list, v_list)):
        if (k is None) != (v is None):
            raise ValueError(f"partition {p}: give both K and V, or neither")
        if k is not None:
            _check_kv(k, v, s.B, s.H, s.D, cache.dtype, f"partition {p}")
            _same_device("dita_attn_step", q, k, v)
    if o is None:
        o = torch.empty(so, dtype=cache.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(sl, dtype=torch.float32, device=q.device)
    _expect(o, so, cache.dtype, "o")
    _expect(lse, sl, torch.float32, "lse")
    _same_device("dita_attn_step", cache.buffer, q, o, lse)
    nk = (ctypes.c_int64 * P)(*[(k.shape[2] if k is not None else 0) for k in k_list])
    info = StepInfo()
    if events is not None:
        info.ev_begin, info.ev_attn_end, info.ev_end = events
    m = (ctypes.c_uint8 * P).from_buffer_copy(mask.tobytes())
    args = (cache.handle, _ptr(q), _ptr_array([_ptr(k) for k in k_list]),
            _ptr_array([_ptr(v) for v in v_list]), nk, m, step, _ptr(o), _ptr(lse),
            _stream(q, stream))
    if side_stream is None and compose_next is None:
        _check(_lib.dita_attn_step(*args, ctypes.byref(info)), "dita_attn_step")
    else:
        nxt = None
        if compose_next is not None:
            nm = np.ascontiguousarray(np.asarray(compose_next, dtype=np.uint8))
            if nm.shape != (P,):
                raise ValueError("compose_next must have P entries")
            nxt = (ctypes.c_uint8 * P).from_buffer_copy(nm.tobytes())
        opts = StepOpts(side_stream.cuda_stream if side_stream is not None else None,
                        int(min_premerge), 0,
                        ctypes.cast(nxt, ctypes.POINTER(ctypes.c_uint8)) if nxt is not None else None)
        _check(_lib.dita_attn_step_ex(*args, ctypes.byref(opts), ctypes.byref(info)),
               "dita_attn_step_ex")
    return o, lse, info


def dita_state_contrib(lse_list: Sequence, lse, w=None, stream=None):
    """Device float64 [P]: mean over rows of exp(LSE_p - LSE) for each state's LSE."""
    torch = _torch()
    P = len(lse_list)
    if lse.dim() != 3:
        raise ValueError(f"lse must be [B, H, Nq], got shape {tuple(lse.shape)}")
    B, H, Nq = lse.shape
    _expect(lse, lse.shape, torch.float32, "lse")
    for i, x in enumerate(lse_list):
        _expect(x, lse.shape, torch.float32, f"lse_list[{i}]")
    if w is None:
        w = torch.empty(P, dtype=torch.float64, device=lse.device)
    _expect(w, (P,), torch.float64, "w")
    _same_device("dita_state_contrib", lse, *lse_list, w)
    shape = Shape(B, H, 64, DITA_F32, Nq, 0.0)   # only B, H, Nq matter here
    _check(_lib.dita_state_contrib(ctypes.byref(shape), P, _ptr_array([_ptr(x) for x in lse_list]),
                                   _ptr(lse), _ptr(w), _stream(lse, stream)), "dita_state_contrib")
    return w


def dita_state_change(o_new, o_prev, lse_new=None, lse_prev=None, roll: bool = False, out=None,
                      stream=None):
    """Device float64 [3]: sum (new - prev)^2, sum prev^2 and the relative change
    sqrt of their ratio; with ``roll`` the new state is also copied over prev."""
    torch = _torch()
    if o_new.dim() != 4:
        raise ValueError(f"states must be [B, H, Nq, D], got shape {tuple(o_new.shape)}")
    _expect(o_prev, o_new.shape, o_new.dtype, "o_prev")
    if roll and (lse_new is None or lse_prev is None):
        raise ValueError("rolling needs lse_new and lse_prev")
    for t, name in ((lse_new, "lse_new"), (lse_prev, "lse_prev")):
        if t is not None:
            _expect(t, o_new.shape[:3], torch.float32, name)
    if out is None:
        out = torch.empty(3, dtype=torch.float64, device=o_new.device)
    _expect(out, (3,), torch.float64, "out")
    _same_device("dita_state_change", o_new, o_prev, lse_new, lse_prev, out)
    shape = make_shape(o_new)
    _check(_lib.dita_state_change(ctypes.byref(shape), _ptr(o_new), _ptr(lse_new), _ptr(o_prev),
                                  _ptr(lse_prev), int(bool(roll)), _ptr(out), _stream(o_new, stream)),
           "dita_state_change")
    return out


def dita_state_change_noalloc(o_new, o_prev, out, lse_new=None, lse_prev=None,
                              roll: bool = False, stream=None):
    """dita_state_change without any device allocation: the caller passes ``out``
    (float64 [3]); the library's fixed device scratch holds the partial sums, so
    calls that overlap on one GPU race."""
    torch = _torch()
    if o_new.dim() != 4:
        raise ValueError(f"states must be [B, H, Nq, D], got shape {tuple(o_new.shape)}")
    _expect(o_prev, o_new.shape, o_new.dtype, "o_prev")
    if roll and (lse_new is None or lse_prev is None):
        raise ValueError("rolling needs lse_new and lse_prev")
    for t, name in ((lse_new, "lse_new"), (lse_prev, "lse_prev")):
        if t is not None:
            _expect(t, o_new.shape[:3], torch.float32, name)
    _expect(out, (3,), torch.float64, "out")
    _same_device("dita_state_change_noalloc", o_new, o_prev, lse_new, lse_prev, out)
    shape = make_shape(o_new)
    _check(_lib.dita_state_change_noalloc(ctypes.byref(shape), _ptr(o_new), _ptr(lse_new),
                                          _ptr(o_prev), _ptr(lse_prev), int(bool(roll)), _ptr(out),
                                          _stream(o_new, stream)), "dita_state_change_noalloc")
    return out


class ErrorPlanner:
    """The library's error-guided, group-wise planner (dita_planner_*)."""

    def __init__(self, P: int, q: int, group_size: int, budget: float, anchor_period: int = 0,
                 fresh_weight: float = 0.0):
        self.P = P
        h = ctypes.c_void_p()
        _check(_lib.dita_planner_create(ctypes.byref(h), ctypes.byref(
            ErrorPlan(P, q, group_size, anchor_period, float(budget), float(fresh_weight)))),
            "dita_planner_create")
        self.handle = h.value

    def set_weights(self, w: Sequence[float]):
        arr = (ctypes.c_double * self.P)(*[float(x) for x in w])
        _check(_lib.dita_planner_set_weights(self.handle, arr), "dita_planner_set_weights")

    def observe(self, step: int, change: float):
        _check(_lib.dita_planner_observe(self.handle, step, float(change)), "dita_planner_observe")

    def mask(self, step: int, valid=None, stamp=None, cache: Optional["StateCache"] = None):
        """(reuse uint8[P], estimated error float64[P]); metadata from ``cache`` or the arrays."""
        out = (ctypes.c_uint8 * self.P)()
        err = (ctypes.c_double * self.P)()
        if cache is not None:
            _check(_lib.dita_planner_mask_cache(self.handle, cache.handle, step, out, err),
                   "dita_planner_mask_cache")
        else:
            v = (ctypes.c_uint8 * self.P)(*[int(x) for x in valid])
            t = (ctypes.c_int64 * self.P)(*[int(x) for x in stamp])
            _check(_lib.dita_planner_mask(self.handle, step, v, t, out, err), "dita_planner_mask")
        return (np.frombuffer(bytes(out), dtype=np.uint8).copy(),
                np.frombuffer(bytes(err), dtype=np.float64).copy())

    def close(self):
        if self.handle:
            _lib.dita_planner_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Event:
    """A raw HIP event (for timing kernels on the stream they run on)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(_lib.dita_event_create(ctypes.byref(h)), "dita_event_create")
        self.handle = h.value

    def record(self, stream=None):
        torch = _torch()
        st = (stream or torch.cuda.current_stream()).cuda_stream
        _check(_lib.dita_event_record(self.handle, st), "dita_event_record")

    def elapsed_ms(self, later: "Event") -> float:
        ms = ctypes.c_float()
        _check(_lib.dita_event_elapsed_ms(self.handle, later.handle, ctypes.byref(ms)),
               "dita_event_elapsed_ms")
        return ms.value

    def __del__(self):
        try:
            if self.handle:
                _lib.dita_event_destroy(self.handle)
        except Exception:
            pass
