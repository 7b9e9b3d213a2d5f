"""Thin ctypes binding of libmoe.so (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the MoE layer runs in the library's
HIP kernels.  Tensors are torch device tensors (PyTorch supplies device memory
and streams); functions take an optional ``stream`` (a torch.cuda.Stream,
default: the current stream).  If the library is not built, or a call returns
an error status, a RuntimeError is raised -- there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_HIP = 3
MOE_ERR_NO_MEMORY = 4
MOE_ERR_CACHE_CAPACITY = 5
MOE_DT_F32, MOE_DT_BF16, MOE_DT_F16 = 0, 1, 2
MOE_WFMT_I4B32, MOE_WFMT_I8B32 = 4, 8
MOE_ACT_FLOAT, MOE_ACT_Q8 = 0, 1

EXPORTED = [
    "moe_version", "moe_last_hip_error", "moe_status_string", "moe_expert_bytes", "moe_pack_experts",
    "moe_unpack_experts", "moe_workspace_size", "moe_route", "moe_route_permute", "moe_permute", "moe_quantize_act",
    "moe_expert_ffn", "moe_expert_ffn_combine", "moe_expert_ffn_combine_slots", "moe_route_ffn_combine_slots",
    "moe_route_ffn_combine_slots_noalloc", "moe_host_pool_create", "moe_host_pool_destroy", "moe_host_expert_ffn",
    "moe_rmsnorm",
    "moe_combine", "moe_cache_create", "moe_cache_destroy", "moe_cache_set_resident", "moe_cache_lookup",
    "moe_cache_stage", "moe_cache_set_stage_mode", "moe_cache_set_stage_fault_hook", "moe_cache_map_host", "moe_usage_accumulate", "moe_cache_plan", "moe_cache_replace",
]


MOE_STAGE_MEMCPY = 0
MOE_STAGE_KERNEL = 1

# int hook(void* user, int layer, int index, int expert): nonzero fails the staging call
STAGE_FAULT_FN = C.CFUNCTYPE(C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_int)

# device scratch of moe_route_ffn_combine_slots_noalloc (include/moe.h)
MOE_NOALLOC_SCRATCH_BYTES = 2 << 20


class MoeError(RuntimeError):
    def __init__(self, fn, status, hip_err):
        self.status = status
        self.hip_error = hip_err
        super().__init__("%s failed: status %d (%s), hipError %d" % (fn, status, _status_name(status), hip_err))


class FfnArgs(C.Structure):
    _fields_ = [
        ("T", C.c_int), ("d", C.c_int), ("f", C.c_int), ("E", C.c_int), ("k", C.c_int),
        ("wfmt", C.c_int), ("act_mode", C.c_int),
        ("x", C.c_void_p), ("x_dtype", C.c_int),
        ("xq", C.c_void_p), ("sx", C.c_void_p),
        ("expert_ptrs", C.c_void_p),
        ("counts", C.c_void_p), ("offsets", C.c_void_p), ("sorted_idx", C.c_void_p), ("active", C.c_void_p),
        ("y_perm", C.c_void_p), ("y_dtype", C.c_int),
        ("shared_blob", C.c_void_p), ("y_shared", C.c_void_p),
        ("ws", C.c_void_p), ("ws_bytes", C.c_size_t),
        ("phase", C.c_int),
    ]


_lib = None


def lib():
    """Load libmoe.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so not built: run `python -m sparse_moe_expert_gemv_amd.build` "
                               "(or __graft_entry__.build()) first")
        L = C.CDLL(LIB_PATH)
        P, I, S = C.c_void_p, C.c_int, C.c_size_t
        sig = {
            "moe_version": ([], I), "moe_last_hip_error": ([], I), "moe_status_string": ([I], C.c_char_p),
            "moe_expert_bytes": ([I, I, I], S),
            "moe_pack_experts": ([P, P, I, I, I, I, P], I), "moe_unpack_experts": ([P, P, I, I, I, I, P], I),
            "moe_workspace_size": ([I, I, I, I, I, I, C.POINTER(S)], I),
            "moe_route": ([P, I, I, I, P, P, I, I, P, P, P, S, P], I),
            "moe_permute": ([P, I, I, I, P, P, P, P, P, P, S, P], I),
            "moe_route_permute": ([P, I, I, I, P, P, I, I, P, P, P, P, P, P, P, P, S, P], I),
            "moe_quantize_act": ([P, I, I, I, P, P, P], I),
            "moe_rmsnorm": ([P, I, I, C.c_float, P, P], I),
            "moe_expert_ffn": ([C.POINTER(FfnArgs), P], I),
            "moe_expert_ffn_combine": ([C.POINTER(FfnArgs), P, P, P, P, P, P], I),
            "moe_expert_ffn_combine_slots": ([C.POINTER(FfnArgs), P, P, P, P, P], I),
            "moe_route_ffn_combine_slots": ([C.POINTER(FfnArgs), P, P, P, P, P, P, P], I),
            "moe_route_ffn_combine_slots_noalloc": ([C.POINTER(FfnArgs), P, P, P, P, P, P, P], I),
            "moe_host_pool_create": ([I, C.POINTER(P)], I),
            "moe_host_pool_destroy": ([P], I),
            "moe_host_expert_ffn": ([P, I, P, P, P, I, I, I, I, P, P], I),
            "moe_combine": ([P, I, P, P, P, P, I, I, I, P, P], I),
            "moe_cache_create": ([C.POINTER(P), I, I, I, S, P, P, I, I], I),
            "moe_cache_destroy": ([P], I),
            "moe_cache_set_resident": ([P, P, I, P, P], I),
            "moe_cache_lookup": ([P, I, P, C.POINTER(I), P, C.POINTER(I)], I),
            "moe_cache_stage": ([P, I, I, P, P, P, P], I),
            "moe_cache_set_stage_mode": ([P, I, I], I),
            "moe_cache_set_stage_fault_hook": ([P, STAGE_FAULT_FN, P], I),
            "moe_cache_map_host": ([P, I, P, P, P, P], I),
            "moe_usage_accumulate": ([P, P, I, P], I),
            "moe_cache_plan": ([I, P, P, I, C.c_float, P, P, C.POINTER(I)], I),
            "moe_cache_replace": ([P, I, P, P, P, P, P], I),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _status_name(st):
    try:
        return lib().moe_status_string(st).decode()
    except Exception:  # noqa: BLE001 - only used for messages
        return "?"


def _check(name, st):
    if st != MOE_OK:
        raise MoeError(name, st, lib().moe_last_hip_error())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _xdtype(t):
    import torch
    if t.dtype == torch.float32:
        return MOE_DT_F32
    if t.dtype == torch.bfloat16:
        return MOE_DT_BF16
    raise ValueError("hidden states must be float32 or bfloat16, got %s" % t.dtype)


def _ydtype(t):
    import torch
    return {torch.float32: MOE_DT_F32, torch.float16: MOE_DT_F16}[t.dtype]


# ---------------------------------------------------------------- calls ----

def moe_version() -> int:
    return lib().moe_version()


def moe_expert_bytes(wfmt: int, d: int, f: int) -> int:
    return int(lib().moe_expert_bytes(wfmt, d, f))


def moe_workspace_size(T, d, f, E, k, act_mode) -> int:
    out = C.c_size_t(0)
    _check("moe_workspace_size", lib().moe_workspace_size(T, d, f, E, k, act_mode, C.byref(out)))
    return out.value


def moe_pack_experts(src, dst, n, wfmt, d, f, stream=None):
    _check("moe_pack_experts", lib().moe_pack_experts(_ptr(src), _ptr(dst), n, wfmt, d, f, _stream(stream)))


def moe_unpack_experts(src, dst, n, wfmt, d, f, stream=None):
    _check("moe_unpack_experts", lib().moe_unpack_experts(_ptr(src), _ptr(dst), n, wfmt, d, f, _stream(stream)))


def moe_route(x, Wr, bias, k, ids, gates, ws, stream=None):
    T, d = x.shape
    E = Wr.shape[0]
    _check("moe_route", lib().moe_route(_ptr(x), _xdtype(x), T, d, _ptr(Wr), _ptr(bias), E, k, _ptr(ids),
                                        _ptr(gates), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_route_permute(x, Wr, bias, k, ids, gates, counts, offsets, sorted_idx, dest, active, ws, stream=None):
    T, d = x.shape
    E = Wr.shape[0]
    _check("moe_route_permute", lib().moe_route_permute(
        _ptr(x), _xdtype(x), T, d, _ptr(Wr), _ptr(bias), E, k, _ptr(ids), _ptr(gates), _ptr(counts), _ptr(offsets),
        _ptr(sorted_idx), _ptr(dest), _ptr(active), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_permute(ids, E, counts, offsets, sorted_idx, dest, active, ws, stream=None):
    T, k = ids.shape
    _check("moe_permute", lib().moe_permute(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(sorted_idx),
                                            _ptr(dest), _ptr(active), _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream)))


def moe_rmsnorm(x, out, eps=1e-6, stream=None):
    T, d = x.shape
    _check("moe_rmsnorm", lib().moe_rmsnorm(_ptr(x), T, d, eps, _ptr(out), _stream(stream)))


def moe_quantize_act(x, xq, sx, stream=None):
    T, d = x.shape
    _check("moe_quantize_act", lib().moe_quantize_act(_ptr(x), _xdtype(x), T, d, _ptr(xq), _ptr(sx),
                                                      _stream(stream)))


def _ffn_args(T, d, f, E, k, wfmt, act_mode, expert_ptrs, counts, offsets, sorted_idx, active, y_perm, ws, x, xq,
              sx, shared_blob, y_shared, phase):
    a = FfnArgs()
    a.T, a.d, a.f, a.E, a.k = T, d, f, E, k
    a.wfmt, a.act_mode = wfmt, act_mode
    a.x = None if x is None else x.data_ptr()
    a.x_dtype = MOE_DT_F32 if x is None else _xdtype(x)
    a.xq = None if xq is None else xq.data_ptr()
    a.sx = None if sx is None else sx.data_ptr()
    a.expert_ptrs = expert_ptrs.data_ptr()
    a.counts, a.offsets = counts.data_ptr(), offsets.data_ptr()
    a.sorted_idx, a.active = sorted_idx.data_ptr(), active.data_ptr()
    a.y_perm, a.y_dtype = y_perm.data_ptr(), _ydtype(y_perm)
    a.shared_blob = None if shared_blob is None else shared_blob.data_ptr()
    a.y_shared = None if y_shared is None else y_shared.data_ptr()
    a.ws, a.ws_bytes = ws.data_ptr(), ws.numel() * ws.element_size()
    a.phase = phase
    return a


def moe_expert_ffn(*, T, d, f, E, k, wfmt, act_mode, expert_ptrs, counts, offsets, sorted_idx, active, y_perm,
                   ws, x=None, xq=None, sx=None, shared_blob=None, y_shared=None, stream=None, phase=0):
    a = _ffn_args(T, d, f, E, k, wfmt, act_mode, expert_ptrs, counts, offsets, sorted_idx, active, y_perm, ws, x, xq,
                  sx, shared_blob, y_shared, phase)
    _check("moe_expert_ffn", lib().moe_expert_ffn(C.byref(a), _stream(stream)))


def moe_expert_ffn_combine_slots(*, T, d, f, E, k, wfmt, act_mode, expert_ptrs, ws, ids, gates, out, x,
                                 residual=None, shared_blob=None, stream=None, phase=0):
    a = FfnArgs()
    a.T, a.d, a.f, a.E, a.k = T, d, f, E, k
    a.wfmt, a.act_mode = wfmt, act_mode
    a.x, a.x_dtype = x.data_ptr(), _xdtype(x)
    a.expert_ptrs = expert_ptrs.data_ptr()
    a.shared_blob = None if shared_blob is None else shared_blob.data_ptr()
    a.ws, a.ws_bytes = ws.data_ptr(), ws.numel() * ws.element_size()
    a.y_dtype, a.phase = MOE_DT_F32, phase
    _check("moe_expert_ffn_combine_slots", lib().moe_expert_ffn_combine_slots(
        C.byref(a), _ptr(ids), _ptr(gates), _ptr(residual), _ptr(out), _stream(stream)))


def moe_route_ffn_combine_slots(*, T, d, f, E, k, wfmt, act_mode, expert_ptrs, ws, Wr, bias, ids, gates, out, x,
                                residual=None, shared_blob=None, stream=None, phase=0):
    a = FfnArgs()
    a.T, a.d, a.f, a.E, a.k = T, d, f, E, k
    a.wfmt, a.act_mode = wfmt, act_mode
    a.x, a.x_dtype = x.data_ptr(), _xdtype(x)
    a.expert_ptrs = expert_ptrs.data_ptr()
    a.shared_blob = None if shared_blob is None else shared_blob.data_ptr()
    a.ws, a.ws_bytes = ws.data_ptr(), ws.numel() * ws.element_size()
    a.y_dtype, a.phase = MOE_DT_F32, phase
    _check("moe_route_ffn_combine_slots", lib().moe_route_ffn_combine_slots(
        C.byref(a), _ptr(Wr), _ptr(bias), _ptr(ids), _ptr(gates), _ptr(residual), _ptr(out), _stream(stream)))


def moe_route_ffn_combine_slots_noalloc(*, T, d, f, E, k, wfmt, act_mode, expert_ptrs, Wr, bias, ids, gates, out, x,
                                        residual=None, shared_blob=None, stream=None):
    """The decode layer with the library's own device scratch (no workspace)."""
    a = FfnArgs()
    a.T, a.d, a.f, a.E, a.k = T, d, f, E, k
    a.wfmt, a.act_mode = wfmt, act_mode
    a.x, a.x_dtype = x.data_ptr(), _xdtype(x)
    a.expert_ptrs = expert_ptrs.data_ptr()
    a.shared_blob = None if shared_blob is None else shared_blob.data_ptr()
    a.ws, a.ws_bytes = None, 0
    a.y_dtype, a.phase = MOE_DT_F32, 0
    _check("moe_route_ffn_combine_slots_noalloc", lib().moe_route_ffn_combine_slots_noalloc(
        C.byref(a), _ptr(Wr), _ptr(bias), _ptr(ids), _ptr(gates), _ptr(residual), _ptr(out), _stream(stream)))


def moe_expert_ffn_combine(*, T, d, f, E, k, wfmt, act_mode, expert_ptrs, counts, offsets, sorted_idx, active, y_perm,
                           ws, ids, dest, gates, out, residual=None, x=None, xq=None, sx=None, shared_blob=None,
                           y_shared=None, stream=None):
    a = _ffn_args(T, d, f, E, k, wfmt, act_mode, expert_ptrs, counts, offsets, sorted_idx, active, y_perm, ws, x, xq,
                  sx, shared_blob, y_shared, 0)
    _check("moe_expert_ffn_combine", lib().moe_expert_ffn_combine(C.byref(a), _ptr(ids), _ptr(dest), _ptr(gates),
                                                                  _ptr(residual), _ptr(out), _stream(stream)))


def moe_combine(y_perm, dest, gates, y_shared, residual, out, stream=None):
    T, k = gates.shape
    d = out.shape[1]
    _check("moe_combine", lib().moe_combine(_ptr(y_perm), _ydtype(y_perm), _ptr(dest), _ptr(gates),
                                            _ptr(y_shared), _ptr(residual), T, k, d, _ptr(out), _stream(stream)))


# ---------------------------------------------------------- slot cache ----

class SlotCache:
    """Handle around moe_cache_* (host bookkeeping; device memory is the caller's)."""

    def __init__(self, n_layers, E, n_slots, expert_bytes, dev_pool, dev_staging, n_staging_bufs, staging_slots):
        h = C.c_void_p()
        _check("moe_cache_create", lib().moe_cache_create(C.byref(h), n_layers, E, n_slots, expert_bytes,
                                                          _ptr(dev_pool), _ptr(dev_staging), n_staging_bufs,
                                                          staging_slots))
        self.h = h
        self.E = E

    def set_resident(self, global_ids, host_ptrs, stream=None):
        n = len(global_ids)
        ids = (C.c_int32 * n)(*[int(g) for g in global_ids])
        src = (C.c_void_p * n)(*[int(p) for p in host_ptrs])
        _check("moe_cache_set_resident", lib().moe_cache_set_resident(self.h, ids, n, src, _stream(stream)))

    def lookup(self, layer):
        hit = (C.c_int32 * self.E)()
        miss = (C.c_int32 * self.E)()
        nh, nm = C.c_int(), C.c_int()
        _check("moe_cache_lookup", lib().moe_cache_lookup(self.h, layer, hit, C.byref(nh), miss, C.byref(nm)))
        return list(hit[:nh.value]), list(miss[:nm.value])

    def set_stage_mode(self, mode, n_workgroups=32):
        _check("moe_cache_set_stage_mode", lib().moe_cache_set_stage_mode(self.h, int(mode), int(n_workgroups)))

    def set_stage_fault_hook(self, fn):
        """Install fn(layer, index, expert) -> int, called before each staging copy
        (a nonzero result fails that stage call with that value); None removes it."""
        if fn is None:
            cb = STAGE_FAULT_FN()
        else:
            cb = STAGE_FAULT_FN(lambda _user, layer, index, expert: int(fn(layer, index, expert)))
        _check("moe_cache_set_stage_fault_hook", lib().moe_cache_set_stage_fault_hook(self.h, cb, None))
        self._fault_cb = cb  # the library keeps the pointer: keep the thunk alive

    def stage(self, layer, buf, host_ptrs, dev_table, stream=None, done_event=None):
        """Stage one layer on `stream`; done_event (a torch.cuda.Event) is recorded after it.

        torch creates an event's HIP handle lazily on its first record, so the
        event is recorded here through torch rather than handed to the library.
        """
        import torch
        src = (C.c_void_p * self.E)(*[int(p) for p in host_ptrs])
        st = stream if stream is not None else torch.cuda.current_stream()
        _check("moe_cache_stage", lib().moe_cache_stage(self.h, layer, buf, src, _ptr(dev_table), _stream(st), None))
        if done_event is not None:
            done_event.record(st)

    def map_host(self, layer, host_ptrs, dev_table, stream=None):
        """Point the misses of one layer's table at their pinned host blobs (read in place)."""
        src = (C.c_void_p * self.E)(*[int(p) for p in host_ptrs])
        _check("moe_cache_map_host", lib().moe_cache_map_host(self.h, layer, src, _ptr(dev_table), _stream(stream),
                                                              None))

    def replace(self, evict_ids, admit_ids, host_ptrs_all, dev_tables, stream=None):
        """Swap resident evict_ids[i] for admit_ids[i] (global ids) on `stream`;
        host_ptrs_all is indexed by global id; dev_tables is the [L, E] pointer tables."""
        n = len(evict_ids)
        ev = (C.c_int32 * max(n, 1))(*[int(g) for g in evict_ids])
        ad = (C.c_int32 * max(n, 1))(*[int(g) for g in admit_ids])
        src = (C.c_void_p * len(host_ptrs_all))(*[int(p) for p in host_ptrs_all])
        _check("moe_cache_replace", lib().moe_cache_replace(self.h, n, ev, ad, src, _ptr(dev_tables),
                                                            _stream(stream)))

    def close(self):
        if self.h:
            lib().moe_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass


def moe_usage_accumulate(usage, counts, stream=None):
    """usage[e] += counts[e] on the device (int32 tensors of E entries)."""
    import torch
    assert usage.dtype == torch.int32 and counts.dtype == torch.int32 and usage.numel() == counts.numel()
    _check("moe_usage_accumulate", lib().moe_usage_accumulate(_ptr(usage), _ptr(counts), usage.numel(),
                                                              _stream(stream)))


def moe_cache_plan(resident, score, max_swaps, margin=0.0):
    """Host replacement plan: returns (evict_ids, admit_ids) as int32 numpy arrays."""
    import numpy as np
    res = np.ascontiguousarray(resident, dtype=np.uint8)
    sc = np.ascontiguousarray(score, dtype=np.float32)
    assert res.shape == sc.shape and res.ndim == 1
    ev = np.zeros(max(max_swaps, 1), dtype=np.int32)
    ad = np.zeros(max(max_swaps, 1), dtype=np.int32)
    n = C.c_int()
    _check("moe_cache_plan", lib().moe_cache_plan(res.size, res.ctypes.data, sc.ctypes.data, max_swaps,
                                                  float(margin), ev.ctypes.data, ad.ctypes.data, C.byref(n)))
    return ev[:n.value].copy(), ad[:n.value].copy()


class HostPool:
    """Host threads for moe_host_expert_ffn (the CPU share of missed experts)."""

    def __init__(self, n_threads: int):
        h = C.c_void_p()
        _check("moe_host_pool_create", lib().moe_host_pool_create(int(n_threads), C.byref(h)))
        self.h = h
        self.n_threads = int(n_threads)

    def expert_ffn(self, item_token, item_gate, item_blob_ptrs, wfmt, x, out, d, f):
        """out[item_token[i]] += item_gate[i] * FFN_i(x[item_token[i]]); x, out: fp32 numpy [T, d]
        (out updated in place); item_blob_ptrs: host addresses of canonical blobs."""
        n = len(item_token)
        tok = np.ascontiguousarray(item_token, dtype=np.int32)
        g = np.ascontiguousarray(item_gate, dtype=np.float32)
        ptrs = (C.c_void_p * max(n, 1))(*[int(p) for p in item_blob_ptrs])
        assert x.dtype == np.float32 and out.dtype == np.float32 and x.flags.c_contiguous and out.flags.c_contiguous
        _check("moe_host_expert_ffn", lib().moe_host_expert_ffn(
            self.h, n, tok.ctypes.data_as(C.c_void_p), g.ctypes.data_as(C.c_void_p), C.cast(ptrs, C.c_void_p),
            int(wfmt), int(x.shape[0]), int(d), int(f), x.ctypes.data_as(C.c_void_p),
            out.ctypes.data_as(C.c_void_p)))

    def close(self):
        if self.h:
            lib().moe_host_pool_destroy(self.h)
            self.h = C.c_void_p()
