"""ctypes wrapper of the fp64 CPU oracle (liboracle_kda.so, built from kda_oracle.c).

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py. The GPU library never imports or links it.

All arrays are host numpy arrays in the layouts of include/kda_oracle.h:
q, k [T, H, d_k] and v [T, H, d_v] as uint16 (bf16 bit patterns) or float32;
alpha float32 [T, H] (scalar gate) or [T, H, d_k] (per-key gate); beta float32
[T, H]; initial_state float32 [N, H, d_v, d_k] or None; cu_seqlens int64 [N+1].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "liboracle_kda.so")
# Tests that plant mistakes in a copy of the oracle point this at the copy.
LIB_OVERRIDE = os.environ.get("KDA_ORACLE_LIB")

OK, MISMATCH, ERR_ARG, ERR_DOMAIN = 0, 1, -1, -2


def build(verbose: bool = False) -> str:
    """Compile the oracle with the host C compiler (portable flags: the built
    library also runs on other x86-64 hosts)."""
    cmd = ["gcc", "-O3", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-o", LIB + ".tmp", SRC, "-lpthread", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


class CheckReport(ctypes.Structure):
    _fields_ = [("o_rel", ctypes.c_double), ("final_rel", ctypes.c_double),
                ("snap_rel", ctypes.c_double), ("n_snap", ctypes.c_int64),
                ("threads", ctypes.c_int32), ("nonfinite", ctypes.c_int32),
                ("seconds", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if LIB_OVERRIDE:
            lib = ctypes.CDLL(LIB_OVERRIDE)
        else:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
            lib = ctypes.CDLL(LIB)
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.kda_oracle_snapshot_count.argtypes = [I32, P, I64, P]
        lib.kda_oracle_run.argtypes = [I32, P, I32, I32, I32, I32, I32, I64,
                                       P, P, P, P, P, P, I32, P, P, P]
        lib.kda_recurrent_ref_check.argtypes = [I32, P, I32, I32, I32, I32, I32, I64,
                                                P, P, P, P, P, P, P, P, P, D, D, I32,
                                                P, P, P, P]
        lib.kda_oracle_backward.argtypes = [I32, P, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P,
                                            I32, P, P, P, P, P, P]
        for f in (lib.kda_oracle_snapshot_count, lib.kda_oracle_run, lib.kda_recurrent_ref_check,
                  lib.kda_oracle_backward):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(q, k, v, alpha, beta, cu_seqlens, initial_state):
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if q.dtype not in (np.uint16, np.float32) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must all be uint16 (bf16 bits) or all float32")
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("shape mismatch among q, k, v, beta")
    if alpha.shape == (T, H):
        per_key = 0
    elif alpha.shape == (T, H, dk):
        per_key = 1
    else:
        raise ValueError("alpha must be [T,H] or [T,H,d_k]")
    N = cu.shape[0] - 1
    if cu[-1] != T:
        raise ValueError("cu_seqlens[-1] must equal T")
    init = None
    if initial_state is not None:
        init = np.ascontiguousarray(initial_state, dtype=np.float32)
        if init.shape != (N, H, dv, dk):
            raise ValueError("initial_state must be [N,H,d_v,d_k]")
    return q, k, v, alpha, beta, cu, init, (N, T, H, dk, dv, per_key, int(q.dtype == np.uint16))


def snapshot_count(cu_seqlens, interval: int) -> int:
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    out = ctypes.c_int64(0)
    rc = load().kda_oracle_snapshot_count(cu.shape[0] - 1, _ptr(cu), int(interval), ctypes.byref(out))
    if rc != OK:
        raise ValueError(f"bad cu_seqlens / interval (rc={rc})")
    return out.value


def run(q, k, v, alpha, beta, cu_seqlens, initial_state=None, interval: int = 0,
        threads: int = 0, want_o: bool = True):
    """fp64 reference: returns (o [T,H,dv], final [N,H,dv,dk], snapshots [S,H,dv,dk])."""
    q, k, v, alpha, beta, cu, init, (N, T, H, dk, dv, per_key, is_bf16) = _prep(
        q, k, v, alpha, beta, cu_seqlens, initial_state)
    n_snap = snapshot_count(cu, interval)
    o = np.zeros((T, H, dv), np.float64) if want_o else None
    fin = np.zeros((N, H, dv, dk), np.float64)
    snap = np.zeros((n_snap, H, dv, dk), np.float64)
    rc = load().kda_oracle_run(N, _ptr(cu), H, dk, dv, is_bf16, per_key, int(interval),
                               _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(init),
                               int(threads), _ptr(o), _ptr(fin), _ptr(snap) if n_snap else None)
    if rc != OK:
        raise ValueError(f"oracle rejected its inputs (rc={rc})")
    return o, fin, snap


def ref_check(q, k, v, alpha, beta, cu_seqlens, initial_state=None, interval: int = 0,
              o_cand=None, final_cand=None, snap_cand=None, o_tol: float = 2e-3,
              state_tol: float = 1e-3, threads: int = 0, want_ref: bool = False):
    """Runs kda_recurrent_ref_check. Returns (rc, report dict[, (o_ref, final_ref, snap_ref)])."""
    q, k, v, alpha, beta, cu, init, (N, T, H, dk, dv, per_key, is_bf16) = _prep(
        q, k, v, alpha, beta, cu_seqlens, initial_state)
    n_snap = snapshot_count(cu, interval)

    def f32(a, shape):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=np.float32)
        if a.shape != shape:
            raise ValueError(f"candidate shape {a.shape} != {shape}")
        return a

    o_c = f32(o_cand, (T, H, dv))
    f_c = f32(final_cand, (N, H, dv, dk))
    s_c = f32(snap_cand, (n_snap, H, dv, dk))
    refs = None
    if want_ref:
        refs = (np.zeros((T, H, dv)), np.zeros((N, H, dv, dk)), np.zeros((n_snap, H, dv, dk)))
    rep = CheckReport()
    rc = load().kda_recurrent_ref_check(
        N, _ptr(cu), H, dk, dv, is_bf16, per_key, int(interval), _ptr(q), _ptr(k), _ptr(v),
        _ptr(alpha), _ptr(beta), _ptr(init), _ptr(o_c), _ptr(f_c), _ptr(s_c),
        float(o_tol), float(state_tol), int(threads),
        _ptr(refs[0]) if refs else None, _ptr(refs[1]) if refs else None,
        _ptr(refs[2]) if refs and n_snap else None, ctypes.byref(rep))
    if rc < 0:
        raise ValueError(f"oracle rejected its inputs (rc={rc})")
    out = (rc, rep.as_dict())
    return out + (refs,) if want_ref else out


def backward(q, k, v, alpha, beta, cu_seqlens, initial_state=None, d_o=None, d_final=None,
             threads: int = 0) -> dict:
    """fp64 gradients of sum <d_o, o> + sum <d_final, S_final> (kda_oracle_backward).
    d_o float32 [T, H, d_v]; d_final float32 [N, H, d_v, d_k] or None. Returns a
    dict with dq, dk, dv, dalpha (shaped like alpha), dbeta and d_initial."""
    q, k, v, alpha, beta, cu, init, (N, T, H, dk, dv, per_key, is_bf16) = _prep(
        q, k, v, alpha, beta, cu_seqlens, initial_state)
    d_o = np.ascontiguousarray(np.zeros((T, H, dv)) if d_o is None else d_o, dtype=np.float32)
    if d_o.shape != (T, H, dv):
        raise ValueError("d_o must be [T,H,d_v]")
    dfin = None
    if d_final is not None:
        dfin = np.ascontiguousarray(d_final, dtype=np.float32)
        if dfin.shape != (N, H, dv, dk):
            raise ValueError("d_final must be [N,H,d_v,d_k]")
    out = {"dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
           "dalpha": np.zeros(alpha.shape), "dbeta": np.zeros((T, H)), "d_initial": np.zeros((N, H, dv, dk))}
    rc = load().kda_oracle_backward(N, _ptr(cu), H, dk, dv, is_bf16, per_key, _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(alpha), _ptr(beta), _ptr(init), _ptr(d_o), _ptr(dfin), int(threads),
                                    _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dalpha"]),
                                    _ptr(out["dbeta"]), _ptr(out["d_initial"]))
    if rc != OK:
        raise ValueError(f"oracle rejected its inputs (rc={rc})")
    return out
