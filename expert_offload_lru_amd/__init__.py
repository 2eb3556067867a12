"""MI355X offloaded mixture-of-experts layer with an LRU expert cache.

Thin ctypes binding over the C ABI of ``include/moe_offload.h`` (GPU
library ``libmoe_offload.so``) and ``include/moe_planner.h`` (host slot table,
also built alone as ``libmoe_planner.so`` without HIP).  The binding only
marshals arguments: every step of the layer runs in the native library.
PyTorch tensors are accepted for device memory and streams.

If the GPU library has not been built, importing :class:`Cache` raises: there
is no fallback path.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_offload.so")
# MOE_PLANNER_LIB may name another build of the host slot table (the sanitizer build the
# planner tests run against)
PLANNER_LIB_PATH = os.environ.get("MOE_PLANNER_LIB") or os.path.join(_PKG, "libmoe_planner.so")

# status codes
OK, ERR_INVALID, ERR_CACHE_TOO_SMALL, ERR_OOM, ERR_HIP, ERR_NOT_READY, ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
ERR_IO = -7
# formats
Q_F32, Q_INT4_G32_F16, Q_E2M1_E4M3_G16 = 0, 1, 2
# create flags
POOL_SHARED, SHARED_EXPERT, PREFETCH, WAVES_UNION, POLICY_LFU, ADAPTIVE_CAPACITY = 0x1, 0x2, 0x4, 0x8, 0x10, 0x20
# forward flags
FWD_RESIDUAL = 0x1
DECODE_MAX_TOKENS = 32
# timing mask
TIME_ROUTER, TIME_GATE_UP, TIME_DOWN, TIME_COMBINE, TIME_PREFILL, TIME_FUSED = 0x1, 0x2, 0x4, 0x8, 0x10, 0x20
TIME_GATE_UP_EARLY = 0x40
TIME_DOWN_EARLY = 0x80


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class BucketStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("plans", "hits", "misses", "picks", "pick_hits", "evictions",
                                               "bytes_h2d", "bytes_d2d", "union_sum", "union_max")]


class Stats(ctypes.Structure):
    _fields_ = [("small", BucketStats), ("large", BucketStats), ("prefill", BucketStats),
                ("waves", ctypes.c_uint64), ("forwards", ctypes.c_uint64),
                ("prefetch_issued", ctypes.c_uint64), ("prefetch_used", ctypes.c_uint64),
                ("prefetch_wasted", ctypes.c_uint64), ("prefetch_candidates", ctypes.c_uint64),
                ("prefetch_deferred", ctypes.c_uint64), ("bytes_h2d_copied", ctypes.c_uint64),
                ("bytes_d2d_copied", ctypes.c_uint64), ("host_plan_us", ctypes.c_double),
                ("host_wait_us", ctypes.c_double), ("host_call_us", ctypes.c_double),
                ("host_upload_us", ctypes.c_double), ("host_launch_us", ctypes.c_double),
                ("host_prefetch_us", ctypes.c_double), ("host_event_us", ctypes.c_double),
                ("graph_steps", ctypes.c_uint64), ("ram_hits", ctypes.c_uint64), ("ram_misses", ctypes.c_uint64),
                ("ram_evictions", ctypes.c_uint64), ("bytes_read_file", ctypes.c_uint64)]


_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)


class PlanRecord(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("wave", ctypes.c_int32), ("t0", ctypes.c_int32), ("t1", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("ids", _i32p), ("gate", _f32p), ("slots", _i32p),
                ("n_hits", ctypes.c_int32), ("hits", _i32p), ("n_fills", ctypes.c_int32),
                ("fill_expert", _i32p), ("fill_slot", _i32p), ("n_evictions", ctypes.c_int32),
                ("evict_key", _i64p), ("evict_slot", _i32p)]


TRACE_FN = ctypes.CFUNCTYPE(None, ctypes.POINTER(PlanRecord), ctypes.c_void_p)


class KernelTiming(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_uint64), ("ms", ctypes.c_double), ("bytes", ctypes.c_double),
                ("flops", ctypes.c_double)]


class Timing(ctypes.Structure):
    _fields_ = [(n, KernelTiming) for n in ("router", "gate_up", "down", "combine", "prefill_gemm", "expert_fused",
                                            "gate_up_early", "down_early")]


def _struct_dict(s):
    out = {}
    for name, _t in s._fields_:
        v = getattr(s, name)
        out[name] = _struct_dict(v) if isinstance(v, ctypes.Structure) else v
    return out


def _arr(ptr, n):
    if n <= 0 or not ptr:
        return []
    return [ptr[i] for i in range(n)]


def record_to_dict(r):
    n = (r.t1 - r.t0) * r.top_k
    return dict(layer=r.layer, wave=r.wave, t0=r.t0, t1=r.t1, top_k=r.top_k,
                ids=_arr(r.ids, n), gate=_arr(r.gate, n) if r.gate else None, slots=_arr(r.slots, n),
                hits=_arr(r.hits, r.n_hits),
                fills=list(zip(_arr(r.fill_expert, r.n_fills), _arr(r.fill_slot, r.n_fills))),
                evictions=list(zip(_arr(r.evict_key, r.n_evictions), _arr(r.evict_slot, r.n_evictions))))


def _declare_common(lib):
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    vp, i, u, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    lib.moe_planner_create.argtypes = [i, i, i, i, u, sz, ctypes.POINTER(vp)]
    lib.moe_planner_destroy.argtypes = [vp]
    lib.moe_planner_destroy.restype = None
    lib.moe_planner_decode.argtypes = [vp, i, _i32p, i, _i32p, TRACE_FN, vp, ctypes.POINTER(i)]
    lib.moe_planner_prefill.argtypes = [vp, i, _i32p, i, _i32p, _i32p, ctypes.POINTER(i)]
    lib.moe_planner_order.argtypes = [vp, i, _i32p]
    lib.moe_planner_set_adaptive.argtypes = [vp, i, i, i, i]
    lib.moe_planner_capacity.argtypes = [vp, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.moe_planner_last_runs.argtypes = [vp, _i32p, i, ctypes.POINTER(i)]
    lib.moe_planner_rollback_last.argtypes = [vp]
    lib.moe_planner_stats.argtypes = [vp, ctypes.POINTER(Stats)]


def _declare_gpu(lib):
    vp, i, u, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    lib.moe_expert_bytes.argtypes = [i, i, i]
    lib.moe_expert_bytes.restype = sz
    lib.moe_host_alloc.argtypes = [sz, ctypes.POINTER(vp)]
    lib.moe_host_free.argtypes = [vp]
    lib.moe_cache_create.argtypes = [i, i, i, i, i, i, i, u, ctypes.POINTER(vp)]
    lib.moe_cache_set_layer.argtypes = [vp, i, vp, sz]
    lib.moe_cache_set_expert_ptrs.argtypes = [vp, i, ctypes.POINTER(vp)]
    lib.moe_layer_forward.argtypes = [vp, i, vp, i, vp, vp, vp, vp, u, vp]
    lib.moe_layer_forward_noalloc.argtypes = [vp, i, vp, i, vp, vp, vp, vp, u, vp]
    lib.moe_debug_fail_upload.argtypes = [vp, i]
    lib.moe_stack_forward.argtypes = [vp, vp, i, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp]
    lib.moe_cache_stats.argtypes = [vp, ctypes.POINTER(Stats)]
    lib.moe_cache_reset_stats.argtypes = [vp]
    lib.moe_cache_set_trace.argtypes = [vp, TRACE_FN, vp]
    lib.moe_cache_set_timing.argtypes = [vp, u]
    lib.moe_cache_set_timing_stride.argtypes = [vp, ctypes.c_int]
    lib.moe_cache_set_prefetch.argtypes = [vp, i, i]
    lib.moe_cache_set_decode_fusion.argtypes = [vp, i]
    lib.moe_cache_set_graph.argtypes = [vp, i]
    lib.moe_cache_set_file_store.argtypes = [vp, ctypes.c_char_p, i, i]
    lib.moe_cache_set_adaptive.argtypes = [vp, i, i, i, i]
    lib.moe_cache_set_prelaunch.argtypes = [vp, i]
    lib.moe_cache_layer_capacity.argtypes = [vp, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.moe_cache_timing.argtypes = [vp, ctypes.POINTER(Timing)]
    lib.moe_cache_reset_timing.argtypes = [vp]
    lib.moe_cache_last_routing.argtypes = [vp, _i32p, _f32p, i]
    lib.moe_cache_slot_of.argtypes = [vp, i, i]
    lib.moe_cache_slot_ptr.argtypes = [vp, i, i, ctypes.POINTER(vp)]
    lib.moe_cache_destroy.argtypes = [vp]
    lib.moe_cache_destroy.restype = None
    lib.moe_debug_decode.argtypes = [i, i, vp, i, vp, vp]


_gpu_lib = None
_planner_lib = None


def gpu_lib():
    """The GPU library; raises if it was not built (no fallback)."""
    global _gpu_lib
    if _gpu_lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m expert_offload_lru_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        _declare_common(lib)
        _declare_gpu(lib)
        _gpu_lib = lib
    return _gpu_lib


def planner_lib():
    """The host slot table alone (no HIP)."""
    global _planner_lib
    if _planner_lib is None:
        if not os.path.exists(PLANNER_LIB_PATH):
            raise ImportError(f"{PLANNER_LIB_PATH} is missing: build it with `python -m expert_offload_lru_amd.build`")
        lib = ctypes.CDLL(PLANNER_LIB_PATH)
        _declare_common(lib)
        _planner_lib = lib
    return _planner_lib


def _check(lib, rc):
    if rc != OK:
        raise MoeError(rc, lib.moe_last_error().decode())
    return rc


def _ptr(t):
    """Device/host address of a torch tensor, a numpy array, an int or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    raise TypeError(f"cannot take the address of {type(t)}")


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def expert_bytes(quant, hidden, inter):
    return gpu_lib().moe_expert_bytes(quant, hidden, inter)


class HostBuffer:
    """Pinned, device-mapped host memory from moe_host_alloc, viewable as numpy."""

    def __init__(self, nbytes):
        lib = gpu_lib()
        p = ctypes.c_void_p()
        _check(lib, lib.moe_host_alloc(nbytes, ctypes.byref(p)))
        self.ptr = p.value
        self.nbytes = nbytes

    def numpy(self, dtype=np.uint8, shape=None):
        buf = (ctypes.c_uint8 * self.nbytes).from_address(self.ptr)
        a = np.frombuffer(buf, dtype=np.uint8)
        a = a.view(dtype)
        return a.reshape(shape) if shape is not None else a

    def free(self):
        if self.ptr:
            gpu_lib().moe_host_free(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class Cache:
    """One offloaded-MoE expert cache (moe_cache_create ... moe_cache_destroy)."""

    def __init__(self, n_experts, n_slots, top_k, hidden, inter, quant, n_layers, flags=0):
        self.lib = gpu_lib()
        h = ctypes.c_void_p()
        _check(self.lib, self.lib.moe_cache_create(n_experts, n_slots, top_k, hidden, inter, quant, n_layers, flags,
                                                   ctypes.byref(h)))
        self.h = h.value
        self.E, self.K, self.k, self.H, self.I = n_experts, n_slots, top_k, hidden, inter
        self.quant, self.L, self.flags = quant, n_layers, flags
        self.S = self.lib.moe_expert_bytes(quant, hidden, inter)
        self._trace_cb = None
        self._keep = []

    def set_layer(self, layer, host_store, nbytes=None):
        nbytes = self.E * self.S if nbytes is None else nbytes
        _check(self.lib, self.lib.moe_cache_set_layer(self.h, layer, _ptr(host_store), nbytes))

    def set_expert_ptrs(self, layer, ptrs):
        arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
        _check(self.lib, self.lib.moe_cache_set_expert_ptrs(self.h, layer, arr))

    def forward(self, layer, x, n_tokens, router_w, out, shared_w=None, next_router_w=None, residual=False,
                stream=None):
        _check(self.lib, self.lib.moe_layer_forward(self.h, layer, _ptr(x), n_tokens, _ptr(router_w), _ptr(shared_w),
                                                    _ptr(next_router_w), _ptr(out),
                                                    FWD_RESIDUAL if residual else 0, _stream_handle(stream)))

    def forward_noalloc(self, layer, x, n_tokens, router_w, out, shared_w=None, next_router_w=None, residual=False,
                        stream=None):
        """moe_layer_forward_noalloc: a decode call whose device scratch is the library's static array."""
        _check(self.lib, self.lib.moe_layer_forward_noalloc(self.h, layer, _ptr(x), n_tokens, _ptr(router_w),
                                                            _ptr(shared_w), _ptr(next_router_w), _ptr(out),
                                                            FWD_RESIDUAL if residual else 0, _stream_handle(stream)))

    def forward_rc(self, layer, x, n_tokens, router_w, out, shared_w=None, next_router_w=None, flags=0, stream=None):
        """Same as forward but returns the status code instead of raising."""
        return self.lib.moe_layer_forward(self.h, layer, _ptr(x), n_tokens, _ptr(router_w), _ptr(shared_w),
                                          _ptr(next_router_w), _ptr(out), flags, _stream_handle(stream))

    def stack_forward(self, x, n_tokens, router_ptrs, out, shared_ptrs=None, layer_inputs=None, stream=None):
        """Decode step through all layers (residual chained); router_ptrs/shared_ptrs: device addresses."""
        rp = (ctypes.c_void_p * self.L)(*router_ptrs)
        sp = (ctypes.c_void_p * self.L)(*shared_ptrs) if shared_ptrs is not None else None
        _check(self.lib, self.lib.moe_stack_forward(self.h, _ptr(x), n_tokens, rp, sp, _ptr(out), _ptr(layer_inputs),
                                                    _stream_handle(stream)))

    def stats(self):
        s = Stats()
        _check(self.lib, self.lib.moe_cache_stats(self.h, ctypes.byref(s)))
        return _struct_dict(s)

    def reset_stats(self):
        _check(self.lib, self.lib.moe_cache_reset_stats(self.h))

    def set_trace(self, fn):
        """fn(record dict) per plan, or None."""
        if fn is None:
            self._trace_cb = None
            _check(self.lib, self.lib.moe_cache_set_trace(self.h, TRACE_FN(), None))
            return
        self._trace_cb = TRACE_FN(lambda rec, _u: fn(record_to_dict(rec.contents)))
        _check(self.lib, self.lib.moe_cache_set_trace(self.h, self._trace_cb, None))

    def set_timing(self, mask, stride=1):
        _check(self.lib, self.lib.moe_cache_set_timing_stride(self.h, stride))
        _check(self.lib, self.lib.moe_cache_set_timing(self.h, mask))

    def set_prefetch(self, backlog=4, layers_ahead=3):
        _check(self.lib, self.lib.moe_cache_set_prefetch(self.h, backlog, layers_ahead))

    def set_adaptive(self, period=8, delta=2, pairs=4, floor=None):
        floor = max(self.k, self.K // 2) if floor is None else floor
        _check(self.lib, self.lib.moe_cache_set_adaptive(self.h, period, delta, pairs, floor))

    def layer_capacity(self, layer):
        held, target = ctypes.c_int(), ctypes.c_int()
        _check(self.lib, self.lib.moe_cache_layer_capacity(self.h, layer, ctypes.byref(held), ctypes.byref(target)))
        return held.value, target.value

    def debug_fail_upload(self, nth):
        """The nth upload submission from now fails as if its copy call had failed (-1: none)."""
        _check(self.lib, self.lib.moe_debug_fail_upload(self.h, nth))

    def set_prelaunch(self, on):
        _check(self.lib, self.lib.moe_cache_set_prelaunch(self.h, 1 if on else 0))

    def set_decode_fusion(self, on):
        _check(self.lib, self.lib.moe_cache_set_decode_fusion(self.h, 1 if on else 0))

    def set_file_store(self, path, ram_blocks, n_readers=4):
        """Two-tier store: expert blocks read from `path` into an LRU of pinned RAM blocks (NVMe
        page, "Workflow").  Block (layer, e) sits at byte offset (layer * E + e) * S."""
        _check(self.lib, self.lib.moe_cache_set_file_store(self.h, os.fsencode(path), ram_blocks, n_readers))

    def set_graph(self, on):
        """One-token stack steps as a replayed HIP graph while every expert is resident (SGLang
        page, "What happens with more than one request?"; NVMe page, "Workflow")."""
        _check(self.lib, self.lib.moe_cache_set_graph(self.h, 1 if on else 0))

    def timing(self):
        t = Timing()
        _check(self.lib, self.lib.moe_cache_timing(self.h, ctypes.byref(t)))
        return _struct_dict(t)

    def reset_timing(self):
        _check(self.lib, self.lib.moe_cache_reset_timing(self.h))

    def last_routing(self, n_tokens):
        ids = np.empty((n_tokens, self.k), dtype=np.int32)
        gate = np.empty((n_tokens, self.k), dtype=np.float32)
        _check(self.lib, self.lib.moe_cache_last_routing(self.h, ids.ctypes.data_as(_i32p), gate.ctypes.data_as(_f32p),
                                                         n_tokens))
        return ids, gate

    def slot_of(self, layer, expert):
        return self.lib.moe_cache_slot_of(self.h, layer, expert)

    def slot_ptr(self, layer, slot):
        p = ctypes.c_void_p()
        _check(self.lib, self.lib.moe_cache_slot_ptr(self.h, layer, slot, ctypes.byref(p)))
        return p.value

    def close(self):
        if self.h:
            self.lib.moe_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def debug_decode(quant, what, codes_dev, n, out_dev, stream=None):
    lib = gpu_lib()
    _check(lib, lib.moe_debug_decode(quant, what, _ptr(codes_dev), n, _ptr(out_dev), _stream_handle(stream)))


class Planner:
    """Host slot table alone (libmoe_planner.so, no HIP); same code as the GPU library's."""

    def __init__(self, n_experts, n_slots, top_k, n_layers, flags=0, block_bytes=0, lib=None):
        self.lib = lib or planner_lib()
        h = ctypes.c_void_p()
        _check(self.lib, self.lib.moe_planner_create(n_experts, n_slots, top_k, n_layers, flags, block_bytes,
                                                     ctypes.byref(h)))
        self.h = h.value
        self.E, self.K, self.k, self.L = n_experts, n_slots, top_k, n_layers

    def decode(self, layer, ids):
        """ids int array [b, k] -> (slots [b, k], list of wave records)."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        b = ids.shape[0]
        slots = np.full(ids.shape, -1, dtype=np.int32)
        recs = []
        cb = TRACE_FN(lambda r, _u: recs.append(record_to_dict(r.contents)))
        nw = ctypes.c_int()
        _check(self.lib, self.lib.moe_planner_decode(self.h, layer, ids.ctypes.data_as(_i32p), b,
                                                     slots.ctypes.data_as(_i32p), cb, None, ctypes.byref(nw)))
        return slots, recs

    def decode_rc(self, layer, ids):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        slots = np.full(ids.shape, -1, dtype=np.int32)
        return self.lib.moe_planner_decode(self.h, layer, ids.ctypes.data_as(_i32p), ids.shape[0],
                                           slots.ctypes.data_as(_i32p), TRACE_FN(), None, None)

    def prefill(self, layer, ids):
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
        ex = np.empty(self.E, dtype=np.int32)
        sl = np.empty(self.E, dtype=np.int32)
        n = ctypes.c_int()
        _check(self.lib, self.lib.moe_planner_prefill(self.h, layer, ids.ctypes.data_as(_i32p), ids.size,
                                                      ex.ctypes.data_as(_i32p), sl.ctypes.data_as(_i32p),
                                                      ctypes.byref(n)))
        return ex[:n.value].tolist(), sl[:n.value].tolist()

    def set_adaptive(self, period=8, delta=2, pairs=4, floor=None):
        floor = max(self.k, self.K // 2) if floor is None else floor
        _check(self.lib, self.lib.moe_planner_set_adaptive(self.h, period, delta, pairs, floor))

    def capacity(self, layer):
        held, target = ctypes.c_int(), ctypes.c_int()
        _check(self.lib, self.lib.moe_planner_capacity(self.h, layer, ctypes.byref(held), ctypes.byref(target)))
        return held.value, target.value

    def order(self, layer):
        o = np.empty(self.capacity(layer)[0], dtype=np.int32)
        _check(self.lib, self.lib.moe_planner_order(self.h, layer, o.ctypes.data_as(_i32p)))
        return o.tolist()

    def last_runs(self):
        buf = np.empty(3 * 4096, dtype=np.int32)
        n = ctypes.c_int()
        _check(self.lib, self.lib.moe_planner_last_runs(self.h, buf.ctypes.data_as(_i32p), 4096, ctypes.byref(n)))
        return [tuple(buf[3 * i:3 * i + 3].tolist()) for i in range(n.value)]

    def rollback_last(self):
        _check(self.lib, self.lib.moe_planner_rollback_last(self.h))

    def stats(self):
        s = Stats()
        _check(self.lib, self.lib.moe_planner_stats(self.h, ctypes.byref(s)))
        return _struct_dict(s)

    def close(self):
        if self.h:
            self.lib.moe_planner_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
