"""CPU oracle for the sparse-MoE expert FFN layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never calls it and shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain C99 + OpenMP, double
precision); this module builds it with gcc and marshals numpy arrays.  Every
function takes fp32 hidden states: a bf16 input is passed after exact widening
to fp32.  See the header of ``moe_oracle.c`` for what each step computes and
which passage of the Strata pages it follows.

Parity pins: router ids/ranking (exact rational recomputation, invariants),
gates (closed forms), permutation (brute-force sort), dequantisation
(closed-form blobs, generator round trip), FFN (closed-form identity experts,
dense masked brute force, invariants), Q8 mode (lossless special case, error
bound), combine (linearity, k=1).  All live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

WFMT_I4B32 = 4
WFMT_I8B32 = 8
ACT_FLOAT = 0
ACT_Q8 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
               "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = C.CDLL(_LIB)
        P = C.c_void_p
        i = C.c_int
        lib.orc_half_to_double.argtypes = [C.c_uint16]
        lib.orc_half_to_double.restype = C.c_double
        lib.orc_expert_bytes.argtypes = [i, i, i]
        lib.orc_expert_bytes.restype = C.c_size_t
        lib.orc_dequant_matrix.argtypes = [P, P, i, i, i, P]
        lib.orc_dequant_expert.argtypes = [P, i, i, i, P, P, P]
        lib.orc_route.argtypes = [P, i, i, P, P, i, i, P, P, P]
        lib.orc_permute.argtypes = [P, i, i, i, P, P, P, P]
        lib.orc_quant8.argtypes = [P, i, i, P, P]
        lib.orc_rmsnorm.argtypes = [P, i, i, C.c_double, P]
        lib.orc_expert_ffn.argtypes = [P, i, i, i, P, i, i, P, P, P]
        lib.orc_moe_layer.argtypes = [P, i, i, i, i, i, P, P, P, P, i, i, P, P, i, P, P, P, P, P, P, P]
        lib.orc_num_threads.restype = i
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def num_threads() -> int:
    return _load().orc_num_threads()


def half_to_double(bits: int) -> float:
    return _load().orc_half_to_double(int(bits))


def expert_bytes(wfmt: int, d: int, f: int) -> int:
    return int(_load().orc_expert_bytes(wfmt, d, f))


def dequant_expert(blob: np.ndarray, wfmt: int, d: int, f: int):
    """(Wg [f,d], Wu [f,d], Wd [d,f]) as float64."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    wg = np.empty((f, d)); wu = np.empty((f, d)); wd = np.empty((d, f))
    _check(_load().orc_dequant_expert(_p(blob), wfmt, d, f, _p(wg), _p(wu), _p(wd)), "dequant_expert")
    return wg, wu, wd


def route(x, Wr, bias, k: int, return_logits: bool = False):
    x = _f32(x); Wr = _f32(Wr)
    T, d = x.shape
    E = Wr.shape[0]
    b = None if bias is None else _f32(bias)
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float32)
    logits = np.empty((T, E), dtype=np.float64) if return_logits else None
    _check(_load().orc_route(_p(x), T, d, _p(Wr), _p(b), E, k, _p(ids), _p(gates), _p(logits)), "route")
    return (ids, gates, logits) if return_logits else (ids, gates)


def permute(ids, E: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_idx = np.empty(T * k, dtype=np.int32)
    dest = np.empty(T * k, dtype=np.int32)
    _check(_load().orc_permute(_p(ids), T, k, E, _p(counts), _p(offsets), _p(sorted_idx), _p(dest)), "permute")
    return counts, offsets, sorted_idx, dest


def rmsnorm(x, eps: float = 1e-6):
    x = _f32(x)
    T, d = x.shape
    out = np.empty((T, d), dtype=np.float32)
    _check(_load().orc_rmsnorm(_p(x), T, d, eps, _p(out)), "rmsnorm")
    return out


def quant8(x):
    x = _f32(x)
    rows, K = x.shape
    q = np.empty((rows, K), dtype=np.int8)
    s = np.empty((rows, K // 32), dtype=np.float32)
    _check(_load().orc_quant8(_p(x), rows, K, _p(q), _p(s)), "quant8")
    return q, s


def expert_ffn(X, blob, wfmt: int, f: int, act_mode: int = ACT_FLOAT, return_gu: bool = False):
    X = _f32(X)
    M, d = X.shape
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    Y = np.empty((M, d))
    G = np.empty((M, f)) if return_gu else None
    U = np.empty((M, f)) if return_gu else None
    _check(_load().orc_expert_ffn(_p(X), M, d, f, _p(blob), wfmt, act_mode, _p(Y), _p(G), _p(U)), "expert_ffn")
    return (Y, G, U) if return_gu else Y


def moe_layer(x, Wr, bias, experts, shared, wfmt: int, f: int, k: int, act_mode: int = ACT_FLOAT,
              residual=None, tokens=None):
    """Whole layer.  experts: [E, nbytes] uint8 array or list of E uint8 arrays.

    Returns dict(ids, gates, counts, offsets, sorted_idx, dest, out) where out
    covers ``tokens`` (all tokens when None) in the given order.
    """
    x = _f32(x); Wr = _f32(Wr)
    T, d = x.shape
    E = Wr.shape[0]
    keep = []
    ptrs = (C.c_void_p * E)()
    for e in range(E):
        a = np.ascontiguousarray(experts[e], dtype=np.uint8)
        keep.append(a)
        ptrs[e] = a.ctypes.data
    sh = None if shared is None else np.ascontiguousarray(shared, dtype=np.uint8)
    b = None if bias is None else _f32(bias)
    res = None if residual is None else _f32(residual)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n_tok = T if tok is None else len(tok)
    o = dict(ids=np.empty((T, k), np.int32), gates=np.empty((T, k), np.float32), counts=np.empty(E, np.int32),
             offsets=np.empty(E + 1, np.int32), sorted_idx=np.empty(T * k, np.int32),
             dest=np.empty(T * k, np.int32), out=np.empty((n_tok, d), np.float32))
    _check(_load().orc_moe_layer(_p(x), T, d, f, E, k, _p(Wr), _p(b), C.cast(ptrs, C.c_void_p), _p(sh), wfmt,
                                 act_mode, _p(res), _p(tok), n_tok, _p(o["ids"]), _p(o["gates"]), _p(o["counts"]),
                                 _p(o["offsets"]), _p(o["sorted_idx"]), _p(o["dest"]), _p(o["out"])), "moe_layer")
    return o
