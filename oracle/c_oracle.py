"""ctypes binding and build step for the C fp64 oracle (pkv_oracle.c).

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU baseline.  Building it with gcc is part of the build check;
the product library never loads it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pkv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
DT = {"f32": 0, "bf16": 1, "fp8": 2, "i8": 3, "i4": 4}

_lib = None


# Flags of the sanitizer build (address + undefined behaviour) that the CPU
# tests load in a child process through PKV_ORACLE_LIB, with the sanitizer
# runtime preloaded.
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]


def build(force: bool = True, sanitize: bool = False, out: str | None = None) -> str:
    """Compile pkv_oracle.c with gcc (-O2, plain C, pthreads) into liboracle.so,
    or with ``sanitize`` under ASan + UBSan into ``out``."""
    out = out or LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        flags = SAN_FLAGS if sanitize else ["-O2"]
        subprocess.run(["gcc", *flags, "-std=c99", "-fPIC", "-shared", "-pthread", SRC,
                        "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    return out


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("PKV_ORACLE_LIB") or LIB
        if path == LIB and not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(path)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.orc_decode.argtypes = [vp, i32, vp, vp, i32, vp, vp, vp, i32, vp, i32, i32, i32, i32,
                                 i32, i32, f32, vp, i32, vp, i32]
        L.orc_decode.restype = i32
        L.orc_append.argtypes = [vp, vp, i32, vp, i32, vp, i32, vp, vp, i32, i32, i32, i32]
        L.orc_append.restype = i32
        L.orc_gather.argtypes = [vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, vp, vp]
        L.orc_gather.restype = i32
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = ctypes.c_double
        L.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f64.restype = ctypes.c_double
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)


def decode(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, seq_lens, Hq, P, scale,
           k_scales=None, v_scales=None, pairs=None, nthreads=None):
    """fp64 [B, Hq, D] outputs; with ``pairs`` ([(b, h), ...]) only those rows are filled."""
    q, k_pool, v_pool = _c(q), _c(k_pool), _c(v_pool)
    bt, sl = _c(block_tables, np.int32), _c(seq_lens, np.int32)
    ks, vs = _c(k_scales, np.float32), _c(v_scales, np.float32)
    NP, Hkv, PD = k_pool.shape
    if kv_dtype == "i4":                    # two elements per byte
        PD *= 2
    D = PD // P
    B = len(sl)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    pr = None if pairs is None else np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    n = 0 if pr is None else len(pr)
    nthreads = nthreads or len(os.sched_getaffinity(0))
    rc = lib().orc_decode(_p(q), DT[q_dtype], _p(k_pool), _p(v_pool), DT[kv_dtype], _p(ks), _p(vs),
                          _p(bt), bt.shape[1], _p(sl), B, NP, Hq, Hkv, D, P, float(scale),
                          _p(pr), n, _p(out), int(nthreads))
    if rc:
        raise RuntimeError(f"orc_decode failed ({rc})")
    return out


def append(k_new, v_new, kv_dtype, block_tables, seq_lens, k_pool, v_pool, P):
    """In place, like the GPU append; pools must be C-contiguous numpy arrays."""
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    kn, vn = _c(k_new), _c(v_new)
    bt, sl = _c(block_tables, np.int32), _c(seq_lens, np.int32)
    NP, Hkv, PD = k_pool.shape
    if kv_dtype == "i4":                    # pools hold two elements per byte
        PD *= 2
    rc = lib().orc_append(_p(kn), _p(vn), DT[kv_dtype], _p(bt), bt.shape[1], _p(sl), len(sl),
                          _p(k_pool), _p(v_pool), NP, Hkv, PD // P, P)
    if rc:
        raise RuntimeError(f"orc_append failed ({rc})")


def gather(k_pool, v_pool, kv_dtype, block_tables, seq_lens, P, fill):
    """[B, Hkv, max_pages*P, D] arrays of stored elements; rows >= L hold ``fill``."""
    k_pool, v_pool = _c(k_pool), _c(v_pool)
    bt, sl = _c(block_tables, np.int32), _c(seq_lens, np.int32)
    NP, Hkv, PD = k_pool.shape
    if kv_dtype == "i4":                    # two elements per byte, rows packed too
        PD *= 2
    D = PD // P
    rows = bt.shape[1] * P
    row_len = D // 2 if kv_dtype == "i4" else D
    ko = np.full((len(sl), Hkv, rows, row_len), fill, dtype=k_pool.dtype)
    vo = np.full((len(sl), Hkv, rows, row_len), fill, dtype=k_pool.dtype)
    rc = lib().orc_gather(_p(k_pool), _p(v_pool), DT[kv_dtype], _p(bt), bt.shape[1], _p(sl),
                          len(sl), NP, Hkv, D, P, _p(ko), _p(vo))
    if rc:
        raise RuntimeError(f"orc_gather failed ({rc})")
    return ko, vo
