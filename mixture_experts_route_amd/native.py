"""Thin ctypes binding of libmoe_route.so (include/moe_route.h), argument marshalling only.

Every function has the C entry point's name and takes torch tensors (device memory) or
plain integers; it passes their addresses, sizes and the current HIP stream to the
library and raises :class:`MoeError` on a non-zero status.  Importing this module loads
the native library and raises ImportError when it is missing: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_route.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with `python -m mixture_experts_route_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_EDEVICE, MOE_EFILL = 0, -1, -2, -3, -4, -5, -6
MOE_F32, MOE_BF16 = 0, 1
MOE_DECODE_MAX_TOKENS, MOE_DECODE_MAX_TOKENS_NARROW = 16, 8
DERR_EXPERT_ID, DERR_SLOT, DERR_NOT_RESIDENT, DERR_NAN, DERR_FILL, DERR_DUP_ID, DERR_RANGE = 1, 2, 4, 8, 16, 32, 64

EXPORTS = [
    "moe_expert_blob_bytes", "moe_workspace_bytes", "moe_strerror", "moe_workspace_init",
    "moe_check_device_error", "moe_debug_kernel_events", "moe_debug_dequant", "moe_route", "moe_slot_lookup", "moe_group_tokens",
    "moe_expert_ffn_decode", "moe_expert_ffn_prefill", "moe_layer_forward", "moe_layer_forward_static",
    "moe_pool_create", "moe_pool_destroy", "moe_pool_arm", "moe_pool_serve", "moe_pool_get_stats",
    "moe_pool_get_table", "moe_pool_get_profile", "moe_profile_seed", "moe_pool_lend", "moe_pool_unlend",
    "moe_pool_debug_fail_copies", "moe_prefill_plan_get", "moe_debug_force_prefill_plan",
]


class moe_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("block", ctypes.c_int32),
                ("format", ctypes.c_int32), ("codebook", ctypes.c_int8 * 16)]


MOE_FMT_Q4_0, MOE_FMT_CB4, MOE_FMT_AFFINE4 = 0, 1, 2


class moe_layer_weights(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("router_dtype", ctypes.c_int32), ("router_bias", ctypes.c_void_p),
                ("arena", ctypes.c_void_p), ("slot_stride", ctypes.c_int64), ("n_slots", ctypes.c_int32),
                ("shared_blob", ctypes.c_void_p)]


class moe_doorbell(ctypes.Structure):
    _fields_ = [("host_miss_ids", ctypes.c_void_p), ("host_miss_count", ctypes.c_void_p),
                ("ready", ctypes.c_void_p), ("epoch", ctypes.c_uint32), ("host_step_ids", ctypes.c_void_p)]


class moe_prefill_plan(ctypes.Structure):
    _fields_ = [("item_rows", ctypes.c_int32), ("gate_up_kernel", ctypes.c_int32), ("down_kernel", ctypes.c_int32),
                ("router_rows", ctypes.c_int32)]


MOE_GEMM_PIPE128, MOE_GEMM_PIPE64_DEEP, MOE_GEMM_GENERAL = 0, 1, 2


class moe_pool_stats(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int64), ("selections", ctypes.c_int64), ("misses", ctypes.c_int64),
                ("bytes_h2d", ctypes.c_int64), ("bytes_d2h", ctypes.c_int64)]


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} ({code})")
        self.code = code


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_D = ctypes.POINTER(moe_dims)
_W = ctypes.POINTER(moe_layer_weights)
_B = ctypes.POINTER(moe_doorbell)
_PP = ctypes.POINTER(ctypes.c_void_p)

_sig = {
    "moe_expert_blob_bytes": (_SZ, [_D]),
    "moe_workspace_bytes": (_SZ, [_D, _I]),
    "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_workspace_init": (ctypes.c_int, [_P, _SZ, _P]),
    "moe_check_device_error": (ctypes.c_int, [_P, _P, ctypes.POINTER(ctypes.c_int32)]),
    "moe_debug_dequant": (ctypes.c_int, [_D, _P, _I, _P, _P]),
    "moe_debug_kernel_events": (ctypes.c_int, [_I, _P, _P]),
    "moe_route": (ctypes.c_int, [_D, _P, _I, _I, _P, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_slot_lookup": (ctypes.c_int, [_D, _P, _I, _P, _I, _P, _P, _P, _B, _P, _SZ, _P]),
    "moe_group_tokens": (ctypes.c_int, [_D, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn_decode": (ctypes.c_int, [_D, _W, _P, _P, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn_prefill": (ctypes.c_int, [_D, _W, _P, _P, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_forward": (ctypes.c_int, [_D, _W, _P, _B, _P, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_forward_static": (ctypes.c_int, [_D, _W, _P, _B, _P, _I, _I, _P, _P, _P, _P, _P]),
    "moe_pool_create": (ctypes.c_int, [_D, _P, ctypes.c_int64, _I, _P, _P, _PP, _P, _I, _P, _P, _P, _P, _PP]),
    "moe_pool_destroy": (ctypes.c_int, [_P]),
    "moe_pool_arm": (ctypes.c_int, [_P, _B]),
    "moe_pool_serve": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.POINTER(ctypes.c_int32), ctypes.c_int64]),
    "moe_pool_get_stats": (ctypes.c_int, [_P, ctypes.POINTER(moe_pool_stats)]),
    "moe_pool_get_table": (ctypes.c_int, [_P, _P]),
    "moe_pool_get_profile": (ctypes.c_int, [_P, _P]),
    "moe_profile_seed": (ctypes.c_int, [_P, _I, _I, _P]),
    "moe_pool_lend": (ctypes.c_int, [_P, _I, _P, _P, _PP]),
    "moe_pool_unlend": (ctypes.c_int, [_P, _P]),
    "moe_pool_debug_fail_copies": (ctypes.c_int, [_P, _I]),
    "moe_prefill_plan_get": (ctypes.c_int, [_D, _I, ctypes.POINTER(moe_prefill_plan)]),
    "moe_debug_force_prefill_plan": (ctypes.c_int, [ctypes.POINTER(moe_prefill_plan)]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def strerror(code: int) -> str:
    return _lib.moe_strerror(code).decode()


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoeError(rc, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def dims(hidden: int, ffn: int, n_experts: int, top_k: int, n_shared: int = 1, block: int = 32, format: int = 0,
         codebook=None) -> moe_dims:
    cb = (ctypes.c_int8 * 16)(*([int(v) for v in codebook] if codebook is not None else [0] * 16))
    return moe_dims(hidden, ffn, n_experts, top_k, n_shared, block, format, cb)


def dtype_code(t) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return MOE_BF16
    raise TypeError(f"unsupported activation dtype {t.dtype}")


def layer_weights(router, arena, slot_stride: int, n_slots: int, shared_blob=None, router_bias=None,
                  router_dtype=None) -> moe_layer_weights:
    rd = dtype_code(router) if router_dtype is None else router_dtype
    return moe_layer_weights(_ptr(router), rd, _ptr(router_bias), _ptr(arena), int(slot_stride), int(n_slots),
                             _ptr(shared_blob))


def doorbell(host_miss_ids: int, host_miss_count: int, ready: int, epoch: int) -> moe_doorbell:
    return moe_doorbell(host_miss_ids, host_miss_count, ready, epoch)


def moe_expert_blob_bytes(d: moe_dims) -> int:
    return _lib.moe_expert_blob_bytes(ctypes.byref(d))


def moe_workspace_bytes(d: moe_dims, max_tokens: int) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(d), max_tokens)


def moe_workspace_init(ws, stream=None):
    _check(_lib.moe_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_workspace_init")


def moe_check_device_error(ws, stream=None) -> int:
    bits = ctypes.c_int32(0)
    rc = _lib.moe_check_device_error(_ptr(ws), _stream(stream), ctypes.byref(bits))
    if rc not in (MOE_OK, MOE_EDEVICE):
        _check(rc, "moe_check_device_error")
    return bits.value


TIME_DECODE_GATE_UP, TIME_DECODE_DOWN, TIME_PREFILL_GATE_UP, TIME_PREFILL_DOWN, TIME_DECODE_ROUTE = 1, 2, 3, 4, 5


def moe_debug_kernel_events(which: int, start_event, stop_event):
    _check(_lib.moe_debug_kernel_events(which, start_event, stop_event), "moe_debug_kernel_events")


def moe_debug_dequant(d: moe_dims, blob, matrix: int, out, stream=None):
    _check(_lib.moe_debug_dequant(ctypes.byref(d), _ptr(blob), matrix, _ptr(out), _stream(stream)),
           "moe_debug_dequant")


def moe_route(d: moe_dims, x, n_tokens: int, router, bias, topk_ids, topk_w, logits, ws, stream=None,
              x_dtype=None, router_dtype=None):
    xd = dtype_code(x) if x_dtype is None else x_dtype
    rd = dtype_code(router) if router_dtype is None else router_dtype
    _check(_lib.moe_route(ctypes.byref(d), _ptr(x), xd, n_tokens, _ptr(router), rd, _ptr(bias), _ptr(topk_ids),
                          _ptr(topk_w), _ptr(logits), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_route")


def moe_slot_lookup(d: moe_dims, table, n_slots: int, topk_ids, n_tokens: int, slots, miss_ids, miss_count, ws,
                    bell: moe_doorbell | None = None, stream=None):
    _check(_lib.moe_slot_lookup(ctypes.byref(d), _ptr(table), n_slots, _ptr(topk_ids), n_tokens, _ptr(slots),
                                _ptr(miss_ids), _ptr(miss_count), ctypes.byref(bell) if bell else None, _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "moe_slot_lookup")


def moe_group_tokens(d: moe_dims, topk_ids, n_tokens: int, counts, offsets, perm, ws, stream=None):
    _check(_lib.moe_group_tokens(ctypes.byref(d), _ptr(topk_ids), n_tokens, _ptr(counts), _ptr(offsets), _ptr(perm),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_group_tokens")


def moe_expert_ffn_decode(d: moe_dims, w: moe_layer_weights, table, x, n_tokens: int, topk_ids, topk_w, y, ws,
                          stream=None, x_dtype=None):
    xd = dtype_code(x) if x_dtype is None else x_dtype
    _check(_lib.moe_expert_ffn_decode(ctypes.byref(d), ctypes.byref(w), _ptr(table), _ptr(x), xd, n_tokens,
                                      _ptr(topk_ids), _ptr(topk_w), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)), "moe_expert_ffn_decode")


def moe_expert_ffn_prefill(d: moe_dims, w: moe_layer_weights, table, x, n_tokens: int, topk_ids, topk_w, y, ws,
                           stream=None, x_dtype=None):
    xd = dtype_code(x) if x_dtype is None else x_dtype
    _check(_lib.moe_expert_ffn_prefill(ctypes.byref(d), ctypes.byref(w), _ptr(table), _ptr(x), xd, n_tokens,
                                       _ptr(topk_ids), _ptr(topk_w), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)), "moe_expert_ffn_prefill")


def moe_layer_forward(d: moe_dims, w: moe_layer_weights, table, x, n_tokens: int, y, ws, topk_ids=None,
                      topk_w=None, bell: moe_doorbell | None = None, stream=None, x_dtype=None):
    xd = dtype_code(x) if x_dtype is None else x_dtype
    _check(_lib.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), _ptr(table), ctypes.byref(bell) if bell else None,
                                  _ptr(x), xd, n_tokens, _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)), "moe_layer_forward")


MOE_STATIC_SCRATCH_BYTES = 8 << 20


def moe_layer_forward_static(d: moe_dims, w: moe_layer_weights, table, x, n_tokens: int, y, device_error,
                             topk_ids=None, topk_w=None, bell: moe_doorbell | None = None, stream=None, x_dtype=None):
    """moe_layer_forward on the library's static per-GPU workspace; ``device_error`` is a device
    int32[1] tensor that receives the call's device error bits."""
    xd = dtype_code(x) if x_dtype is None else x_dtype
    _check(_lib.moe_layer_forward_static(ctypes.byref(d), ctypes.byref(w), _ptr(table),
                                         ctypes.byref(bell) if bell else None, _ptr(x), xd, n_tokens, _ptr(y),
                                         _ptr(topk_ids), _ptr(topk_w), _ptr(device_error), _stream(stream)),
           "moe_layer_forward_static")


def raw(name: str):
    """The raw ctypes function (for tests of the C-level validation)."""
    return getattr(_lib, name)


# ---------------------------------------------------------------------------------------------
# slot-pool service (host side)
# ---------------------------------------------------------------------------------------------

def _hiprt():
    lib = ctypes.CDLL("libamdhip64.so.7")
    lib.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
    lib.hipHostFree.argtypes = [ctypes.c_void_p]
    lib.hipStreamCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    lib.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    return lib


def new_stream():
    """A fresh non-blocking HIP stream at the default priority, as a torch stream object.

    A pool's compute stream waits (in-stream) for a value its copy stream writes; the two must
    not share a hardware queue, so they are created here rather than taken from torch's stream
    pool (whose streams share the few hardware queues round-robin).  Free with free_stream."""
    s = ctypes.c_void_p()
    rc = _hiprt().hipStreamCreateWithFlags(ctypes.byref(s), 0x1)
    if rc != 0:
        raise MoeError(MOE_EHIP, f"hipStreamCreateWithFlags = {rc}")
    return torch.cuda.ExternalStream(s.value)


def free_stream(stream):
    torch.cuda.synchronize()
    _hiprt().hipStreamDestroy(stream.cuda_stream)


HIP_HOST_MALLOC_MAPPED, HIP_HOST_MALLOC_COHERENT = 0x2, 0x40000000


class HostBuffer:
    """Pinned host memory: by default device-mapped and coherent (for doorbell words the GPU
    writes and the host polls); ``flags=0`` for bulk copy buffers.  ``.ptr`` is the address both
    sides use; ``.view(dtype)`` a numpy view."""

    def __init__(self, nbytes: int, flags: int = HIP_HOST_MALLOC_MAPPED | HIP_HOST_MALLOC_COHERENT):
        import numpy as np

        self._hip = _hiprt()
        p = ctypes.c_void_p()
        rc = self._hip.hipHostMalloc(ctypes.byref(p), nbytes, flags)
        if rc != 0:
            raise MoeError(MOE_EHIP, f"hipHostMalloc({nbytes}) = {rc}")
        self.ptr, self.nbytes = p.value, nbytes
        self._np = np.ctypeslib.as_array((ctypes.c_uint8 * nbytes).from_address(self.ptr))
        if flags & HIP_HOST_MALLOC_COHERENT:
            self._np[:] = 0

    def view(self, dtype):
        return self._np.view(dtype)

    def free(self):
        if self.ptr:
            self._hip.hipHostFree(self.ptr)
            self.ptr = 0


def moe_pool_create(d: moe_dims, arena, slot_stride: int, n_slots: int, table, initial, host_home, spares,
                    n_spares: int, host_miss_ids: int, host_counts: int, host_step_ids: int, ready):
    """Returns the pool handle (int).  ``initial``: sequence of n_slots expert ids; ``host_home``:
    sequence of E addresses (0 for experts in ``initial``); ``spares``: n_spares pinned buffers at
    slot_stride apart; other pointers as in the header."""
    init = (ctypes.c_int32 * n_slots)(*[int(e) for e in initial])
    homes = (ctypes.c_void_p * len(host_home))(*[int(a) if a else None for a in host_home])
    out = ctypes.c_void_p()
    _check(_lib.moe_pool_create(ctypes.byref(d), _ptr(arena), int(slot_stride), int(n_slots), _ptr(table), init,
                                homes, _ptr(spares), int(n_spares), host_miss_ids, host_counts, host_step_ids, _ptr(ready),
                                ctypes.byref(out)), "moe_pool_create")
    return out.value


def moe_pool_destroy(pool: int):
    _check(_lib.moe_pool_destroy(pool), "moe_pool_destroy")


def moe_pool_arm(pool: int) -> moe_doorbell:
    bell = moe_doorbell()
    _check(_lib.moe_pool_arm(pool, ctypes.byref(bell)), "moe_pool_arm")
    return bell


def moe_pool_serve(pool: int, ws=None, copy_stream=None, n_experts: int = 0, timeout_us: int = 20_000_000,
                   h2d_stream=None):
    """Serves the armed call; returns the fills [(expert, slot, evicted)].  Raises on MOE_EFILL.
    ``copy_stream`` takes the device->host copies, ``h2d_stream`` (None: the same stream) the
    host->device copies, the table and the release."""
    fills = (ctypes.c_int32 * (3 * max(1, n_experts)))()
    n = ctypes.c_int32()
    h2d = h2d_stream.cuda_stream if h2d_stream is not None else None
    _check(_lib.moe_pool_serve(pool, _ptr(ws), _stream(copy_stream), h2d, fills if n_experts else None,
                               ctypes.byref(n), int(timeout_us)), "moe_pool_serve")
    return [(fills[3 * i], fills[3 * i + 1], fills[3 * i + 2]) for i in range(n.value)] if n_experts else n.value


def moe_pool_get_stats(pool: int) -> moe_pool_stats:
    st = moe_pool_stats()
    _check(_lib.moe_pool_get_stats(pool, ctypes.byref(st)), "moe_pool_get_stats")
    return st


def moe_pool_get_table(pool: int, n_experts: int):
    import numpy as np

    out = np.zeros(n_experts, dtype=np.int32)
    _check(_lib.moe_pool_get_table(pool, out.ctypes.data), "moe_pool_get_table")
    return out


def moe_pool_get_profile(pool: int, n_experts: int):
    import numpy as np

    out = np.zeros(n_experts, dtype=np.int64)
    _check(_lib.moe_pool_get_profile(pool, out.ctypes.data), "moe_pool_get_profile")
    return out


def moe_profile_seed(counts, n_slots: int):
    """Initial residency (hottest first) of a pool of ``n_slots`` slots from per-expert counts."""
    import numpy as np

    c = np.ascontiguousarray(counts, dtype=np.int64)
    out = np.zeros(n_slots, dtype=np.int32)
    _check(_lib.moe_profile_seed(c.ctypes.data, len(c), n_slots, out.ctypes.data), "moe_profile_seed")
    return out


def moe_pool_lend(pool: int, n: int, host_bufs: int, stream=None) -> int:
    """Lends the pool's last ``n`` slots; returns the region's device address."""
    region = ctypes.c_void_p()
    _check(_lib.moe_pool_lend(pool, n, host_bufs, _stream(stream), ctypes.byref(region)), "moe_pool_lend")
    return region.value


def moe_pool_unlend(pool: int, stream=None):
    _check(_lib.moe_pool_unlend(pool, _stream(stream)), "moe_pool_unlend")


def moe_pool_debug_fail_copies(pool: int, after_n: int):
    _check(_lib.moe_pool_debug_fail_copies(pool, after_n), "moe_pool_debug_fail_copies")


def moe_prefill_plan_get(d: moe_dims, n_tokens: int) -> moe_prefill_plan:
    p = moe_prefill_plan()
    _check(_lib.moe_prefill_plan_get(ctypes.byref(d), n_tokens, ctypes.byref(p)), "moe_prefill_plan_get")
    return p


def moe_debug_force_prefill_plan(plan: moe_prefill_plan | None):
    _check(_lib.moe_debug_force_prefill_plan(ctypes.byref(plan) if plan is not None else None),
           "moe_debug_force_prefill_plan")
