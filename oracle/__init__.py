"""fp64 CPU oracle for pool-indexed recurrent-state decode (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It wraps ``oracle.c`` (plain scalar fp64 loops) through
ctypes; it shares no code with the GPU library and never calls it.

The recurrence it evaluates, and where it comes from, is stated in the header
of ``oracle.c``. This module only converts inputs to contiguous float64 arrays
(bf16 and fp32 convert exactly) and hands them over.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

__all__ = ["LIGHTNING", "GDN", "KDA", "L2NORM_QK", "BETA_LOGIT", "GATE",
           "GATE_LOWER_BOUND", "build",
           "decode", "replay", "lib_path"]

LIGHTNING, GDN, KDA = 0, 1, 2
L2NORM_QK, BETA_LOGIT = 1, 2
GATE, GATE_LOWER_BOUND = 4, 8

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def lib_path() -> str:
    return _LIB


def build() -> str:
    """Compile oracle.c with gcc (no fast-math) into liboracle.so."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                    "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # LA_ORACLE_LIB points the pins at a deliberately broken oracle build
        # (tests/test_oracle_mutations.py); normally it is unset.
        path = os.environ.get("LA_ORACLE_LIB")
        if not path:
            path = _LIB
            if (not os.path.exists(_LIB)
                    or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = (
            [ctypes.c_int] * 8 + [dp] * 5 + [ctypes.c_int, dp, dp, ip, ip,
                                             dp, dp, ip, ctypes.c_int, ip,
                                             dp, ip, ctypes.c_int, dp, dp,
                                             ctypes.c_double])
        lib.oracle_replay.restype = ctypes.c_int
        lib.oracle_replay.argtypes = (
            [ctypes.c_int] * 5 + [dp, ctypes.c_int, dp, dp, ip, ip, ip, ip,
                                  ctypes.c_int])
        _lib = lib
    return _lib


def _f64(x):
    """Exact conversion to a contiguous float64 numpy array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16/fp32 -> fp64 is exact
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def decode(variant, q, k, v, g, beta, pool, read_idx, write_idx=None,
           flags=0, inter=False, token_slots=None, num_accepted=None,
           factors=False, cu_seqlens=None, max_tokens=None, A_log=None,
           dt_bias=None, lower_bound=None):
    """Run the fp64 recurrence.

    q, k: [B,T,H,K]; v: [B,T,HV,V]; g: Lightning [HV] decay factors or None,
    GDN [B,T,HV], KDA [B,T,HV,K] log-decay; beta: [B,T,HV] or None
    (Lightning); pool: logical [pool_size,HV,V,K]; read_idx/write_idx: [B].
    token_slots: optional [B, >=T] per-token slot table (then read_idx and
    write_idx are ignored and num_accepted [B] is required).
    factors: also return the per-token records [B,T,HV,2K+V] (a | k | err).
    cu_seqlens: optional [B+1] offsets of a variable-length batch; then every
    per-token array is token-packed ([total, ...] in place of [B, T, ...]) and
    T is max_tokens (default: the longest request).
    A_log [HV], dt_bias ([HV] GDN, [HV,K] KDA), lower_bound: the in-kernel
    gate chain (g then holds the raw gate); see oracle.c for the reading.

    Returns a dict with ``out`` [B,T,HV,V], ``pool`` (the pool after the
    call, float64) and ``inter`` ([B,T,HV,V,K] or None).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    g, beta = _f64(g), _f64(beta)
    pool_in = _f64(pool)
    ridx, widx = _i32(read_idx), _i32(write_idx)
    cu = _i32(cu_seqlens)
    if cu is not None:
        # token-packed: view [total, ...] as [1, total, ...] for the checks
        B = cu.shape[0] - 1
        total = q.shape[0]
        T = (int(max_tokens) if max_tokens is not None
             else max(1, int(np.max(np.diff(cu))) if B > 0 else 1))
        lead = (total,)
        H, K = q.shape[1], q.shape[2]
        HV, V = v.shape[1], v.shape[2]
        if k.shape != q.shape or v.shape[0] != total:
            raise ValueError("q/k/v shapes disagree")
    else:
        B, T, H, K = q.shape
        HV, V = v.shape[2], v.shape[3]
        total = 0
        lead = (B, T)
        if k.shape != q.shape or v.shape[:2] != (B, T):
            raise ValueError("q/k/v shapes disagree")
    pool_size = pool_in.shape[0]
    if pool_in.shape[1:] != (HV, V, K):
        raise ValueError("pool shape %s != [pool_size,%d,%d,%d]"
                         % (pool_in.shape, HV, V, K))
    if token_slots is None and (ridx is None or ridx.shape != (B,) or (
            widx is not None and widx.shape != (B,))):
        raise ValueError("index shape")
    if variant != LIGHTNING and (g is None or beta is None):
        raise ValueError("GDN/KDA need g and beta")
    expect_g = {LIGHTNING: (HV,), GDN: lead + (HV,), KDA: lead + (HV, K)}
    if g is not None and g.shape != expect_g[variant]:
        raise ValueError("g shape %s != %s" % (g.shape, expect_g[variant]))
    if beta is not None and variant != LIGHTNING and beta.shape != lead + (HV,):
        raise ValueError("beta shape")
    slots = _i32(token_slots)
    acc = _i32(num_accepted)
    stride = 0
    if slots is not None:
        if slots.ndim != 2 or slots.shape[0] != B or slots.shape[1] < T:
            raise ValueError("token_slots must be [B, >=T]")
        if acc is None or acc.shape != (B,):
            raise ValueError("num_accepted must be [B]")
        stride = slots.shape[1]
        ridx = np.full((B,), -1, dtype=np.int32)
        widx = None
    a_log, dt = _f64(A_log), _f64(dt_bias)
    if a_log is not None or dt is not None:
        flags |= GATE
        if a_log is None or dt is None or a_log.shape != (HV,) or \
                dt.shape != ((HV,) if variant == GDN else (HV, K)):
            raise ValueError("gate chain needs A_log [HV] and dt_bias "
                             "[HV] (GDN) / [HV, K] (KDA)")
    if lower_bound is not None:
        flags |= GATE_LOWER_BOUND
    pool_out = pool_in.copy()
    # NaN until the oracle writes it: a position it skips cannot pass as 0
    out = np.full(lead + (HV, V), np.nan, dtype=np.float64)
    inter_a = (np.full(lead + (HV, V, K), np.nan, dtype=np.float64)
               if inter else None)
    fac = (np.full(lead + (HV, 2 * K + V), np.nan, dtype=np.float64)
           if factors else None)
    dp = ctypes.c_double
    rc = _load().oracle_decode(
        variant, B, T, H, HV, K, V, flags, _ptr(q, dp), _ptr(k, dp),
        _ptr(v, dp), _ptr(g, dp),
        _ptr(beta if variant != LIGHTNING else None, dp), pool_size,
        _ptr(pool_in, dp), _ptr(pool_out, dp), _ptr(ridx, ctypes.c_int32),
        _ptr(widx, ctypes.c_int32), _ptr(out, dp), _ptr(inter_a, dp),
        _ptr(slots, ctypes.c_int32), stride, _ptr(acc, ctypes.c_int32),
        _ptr(fac, dp), _ptr(cu, ctypes.c_int32), total, _ptr(a_log, dp),
        _ptr(dt, dp), float(lower_bound if lower_bound is not None else 0.0))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments (rc=%d)" % rc)
    return {"out": out, "pool": pool_out, "inter": inter_a, "factors": fac}


def replay(factors, pool, read_idx, write_idx, num_tokens, cu_seqlens=None,
           max_tokens=None):
    """Rebuild states from factor records [B,T,HV,2K+V]: request b starts
    from pool[read_idx[b]] and applies its first num_tokens[b] records;
    the result goes to write_idx[b] (None: the read slot). With cu_seqlens
    the records are token-packed [total,HV,2K+V]. Returns the pool after the
    call (float64)."""
    fac = _f64(factors)
    pool_in = _f64(pool)
    ridx, widx, ntok = _i32(read_idx), _i32(write_idx), _i32(num_tokens)
    cu = _i32(cu_seqlens)
    total = 0
    if cu is not None:
        B = cu.shape[0] - 1
        total, HV, R = fac.shape
        T = (int(max_tokens) if max_tokens is not None
             else max(1, int(np.max(np.diff(cu))) if B > 0 else 1))
    else:
        B, T, HV, R = fac.shape
    V, K = pool_in.shape[2], pool_in.shape[3]
    if R != 2 * K + V or pool_in.shape[1] != HV:
        raise ValueError("factor records do not match the pool")
    if ridx.shape != (B,) or ntok.shape != (B,) or (
            widx is not None and widx.shape != (B,)):
        raise ValueError("index shape")
    pool_out = pool_in.copy()
    dp = ctypes.c_double
    rc = _load().oracle_replay(B, T, HV, K, V, _ptr(fac, dp),
                               pool_in.shape[0], _ptr(pool_in, dp),
                               _ptr(pool_out, dp), _ptr(ridx, ctypes.c_int32),
                               _ptr(widx, ctypes.c_int32),
                               _ptr(ntok, ctypes.c_int32),
                               _ptr(cu, ctypes.c_int32), total)
    if rc != 0:
        raise ValueError("oracle_replay rejected its arguments (rc=%d)" % rc)
    return pool_out
