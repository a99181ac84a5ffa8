"""ctypes front end of the fp64 C oracle (test infrastructure only)."""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def oracle_lib_path() -> str:
    return os.path.join(_HERE, "libkda_oracle.so")


def build_oracle() -> str:
    """Compile kda_oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    out = oracle_lib_path()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _lib():
    global _LIB
    if _LIB is None:
        path = oracle_lib_path()
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build_oracle()
        lib = ctypes.CDLL(path)
        lib.kdao_gate.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _dp, _dp, _dp,
                                  ctypes.c_int32, _dp, _dp, _dp]
        lib.kdao_gate.restype = None
        lib.kdao_gate_backward.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _dp,
                                           _dp, _dp, ctypes.c_int32, _dp, _dp, _dp, _dp, _dp,
                                           _dp, _dp]
        lib.kdao_gate_backward.restype = None
        lib.kdao_prefill_backward.argtypes = [ctypes.c_int32, _ip, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, _dp, _dp, _dp, _dp, _dp,
                                              ctypes.c_double, _dp, _dp, _dp, _dp, _dp, _dp,
                                              _dp, _dp, _dp, ctypes.c_int32]
        lib.kdao_prefill_backward.restype = ctypes.c_int32
        lib.kdao_prefill.argtypes = [ctypes.c_int32, _ip, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, _dp, _dp, _dp, _dp, _dp, ctypes.c_double,
                                     _dp, _dp, _dp, ctypes.c_int32]
        lib.kdao_prefill.restype = ctypes.c_int32
        lib.kdao_decode.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, _dp, _dp, _dp, _dp, _dp, ctypes.c_double,
                                    _dp, _dp, ctypes.c_int32]
        lib.kdao_decode.restype = ctypes.c_int32
        _LIB = lib
    return _LIB


def f64(a) -> np.ndarray:
    """Exact upcast to a C-contiguous fp64 numpy array (bf16/fp32/fp64 in)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_dp)


def gate(x, b, A_log, dt_bias):
    """g = -exp(A_log) softplus(x + dt_bias[h,c]); beta = sigmoid(b). fp64.

    A_log is per head, [H], or per (head, channel), [H, d]: the per-channel
    form is the variant the Kimi K3 artifact audit (§5.2) leaves open for the
    checkpoint's A_log; it is taken only when given explicitly as [H, d]."""
    x, b, A_log, dt_bias = f64(x), f64(b), f64(A_log), f64(dt_bias)
    T, H, d = x.shape
    if A_log.shape not in ((H,), (H, d)) or b.shape != (T, H) or dt_bias.size != H * d:
        raise ValueError("gate: shape mismatch")
    g = np.empty_like(x)
    beta = np.empty_like(b)
    _lib().kdao_gate(T, H, d, _p(x), _p(b), _p(A_log), int(A_log.ndim == 2), _p(dt_bias), _p(g),
                     _p(beta))
    return g, beta


def gate_backward(x, b, A_log, dt_bias, dg, dbeta):
    """Gradient of gate() against dg [T,H,d] and dbeta [T,H], fp64.

    Returns (dx [T,H,d], db [T,H], dA_log (A_log's shape), ddt_bias [H,d])."""
    x, b, A_log, dt_bias = f64(x), f64(b), f64(A_log), f64(dt_bias)
    dg, dbeta = f64(dg), f64(dbeta)
    T, H, d = x.shape
    if A_log.shape not in ((H,), (H, d)) or b.shape != (T, H) or dt_bias.size != H * d \
            or dg.shape != (T, H, d) or dbeta.shape != (T, H):
        raise ValueError("gate_backward: shape mismatch")
    dx = np.empty_like(x)
    db = np.empty_like(b)
    dA = np.empty_like(A_log)
    ddt = np.empty((H, d))
    _lib().kdao_gate_backward(T, H, d, _p(x), _p(b), _p(A_log), int(A_log.ndim == 2),
                              _p(dt_bias), _p(dg), _p(dbeta), _p(dx), _p(db), _p(dA), _p(ddt))
    return dx, db, dA, ddt


def prefill(q, k, v, g, beta, cu_seqlens, initial_state=None, scale=1.0, nthreads=0,
            return_threads=False):
    """Token-by-token fp64 recurrence over packed varlen sequences.

    Returns (o [T,H,dv], final_state [N,H,dk,dv]) as fp64 numpy arrays.
    """
    q, k, v, g, beta = f64(q), f64(k), f64(v), f64(g), f64(beta)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.size - 1
    if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) \
            or beta.shape != (T, H) or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("prefill: bad shapes or cu_seqlens")
    S0 = None if initial_state is None else f64(initial_state)
    if S0 is not None and S0.shape != (N, H, dk, dv):
        raise ValueError("prefill: initial_state shape")
    o = np.zeros((T, H, dv))
    Sf = np.zeros((N, H, dk, dv))
    used = _lib().kdao_prefill(N, cu.ctypes.data_as(_ip), H, dk, dv, _p(q), _p(k), _p(v),
                               _p(g), _p(beta), float(scale), _p(S0), _p(o), _p(Sf),
                               int(nthreads))
    return (o, Sf, used) if return_threads else (o, Sf)


def prefill_backward(q, k, v, g, beta, cu_seqlens, initial_state=None, scale=1.0, d_o=None,
                     dS_final=None, nthreads=0):
    """Gradients of prefill's outputs (o, final state) against d_o [T,H,dv] and
    dS_final [N,H,dk,dv] (either may be None: zero), by reverse-mode through the
    token recurrence in fp64 (kdao_prefill_backward).

    Returns (dq, dk, dv, dg, dbeta, dS0) as fp64 numpy arrays; dS0 is the
    gradient of the initial state (the zero state when none is given)."""
    q, k, v, g, beta = f64(q), f64(k), f64(v), f64(g), f64(beta)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.size - 1
    if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) \
            or beta.shape != (T, H) or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("prefill_backward: bad shapes or cu_seqlens")
    S0 = None if initial_state is None else f64(initial_state)
    dO = None if d_o is None else f64(d_o)
    dSf = None if dS_final is None else f64(dS_final)
    if (S0 is not None and S0.shape != (N, H, dk, dv)) or \
            (dSf is not None and dSf.shape != (N, H, dk, dv)) or \
            (dO is not None and dO.shape != (T, H, dv)):
        raise ValueError("prefill_backward: shape mismatch")
    out = [np.zeros((T, H, dk)), np.zeros((T, H, dk)), np.zeros((T, H, dv)),
           np.zeros((T, H, dk)), np.zeros((T, H)), np.zeros((N, H, dk, dv))]
    _lib().kdao_prefill_backward(N, cu.ctypes.data_as(_ip), H, dk, dv, _p(q), _p(k), _p(v),
                                 _p(g), _p(beta), float(scale), _p(S0), _p(dO), _p(dSf),
                                 *[_p(a) for a in out], int(nthreads))
    return tuple(out)


def decode(q, k, v, g, beta, state, scale=1.0, nthreads=0, return_threads=False):
    """One token per sequence.  Returns (o [N,H,dv], new_state [N,H,dk,dv])."""
    q, k, v, g, beta = f64(q), f64(k), f64(v), f64(g), f64(beta)
    S = f64(state).copy()
    N, H, dk = q.shape
    dv = v.shape[2]
    if S.shape != (N, H, dk, dv) or beta.shape != (N, H):
        raise ValueError("decode: shape mismatch")
    o = np.zeros((N, H, dv))
    used = _lib().kdao_decode(N, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                              float(scale), _p(S), _p(o), int(nthreads))
    return (o, S, used) if return_threads else (o, S)
