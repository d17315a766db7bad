"""Builds tests/sched_host.cpp (the schedule header csrc/sched.hpp, host only)
with the host C++ compiler and loads it with ctypes, once per process."""
import ctypes
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "post_weight_quantization_04_amd", "csrc")
_lib = None

i64, i32 = ctypes.c_int64, ctypes.c_int
p64, p32 = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int)


def load():
    global _lib
    if _lib is not None:
        return _lib
    out = os.path.join(tempfile.mkdtemp(prefix="gptq_sched_"), "libsched_host.so")
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-shared", "-fPIC", "-I", CSRC,
           os.path.join(HERE, "sched_host.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    lib = ctypes.CDLL(out)
    sigs = {
        "chol_rest_tiles": (i64, [i32, i32]),
        "chol_rest_tile": (None, [i32, i64, p64, p64]),
        "chol_paired_default": (i32, [i32]),
        "chol_launch_geom": (None, [i32, i32, i32, p64]),
        "far_split_c": (i32, [i64, i32, i32, i64, i32, p64]),
        "far_units_c": (None, [i64, i32, i32, i64, i32, i32, p64, p64]),
        "far_sub_c": (None, [i64, i32, i32, i64, i32, i64, i64, i64, p64]),
        "far_constants": (i32, [p32, p32, p32]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def chol_geom(k, T, paired):
    out = (ctypes.c_int64 * 3)()
    load().chol_launch_geom(k, T, int(paired), out)
    return {"nchain": out[0], "n_rest": out[1], "grid": out[2]}


def chol_rest_tiles(k, T):
    return load().chol_rest_tiles(k, T)


def chol_rest_tile(k, b):
    i, j = ctypes.c_int64(), ctypes.c_int64()
    load().chol_rest_tile(k, b, ctypes.byref(i), ctypes.byref(j))
    return i.value, j.value


def far_split(n_units, n_sweep, n_cu, c_begin, nstrip):
    out = (ctypes.c_int64 * 4)()
    nf = load().far_split_c(n_units, n_sweep, n_cu, c_begin, nstrip, out)
    return nf, {"n_units": out[0], "per_sweep": out[1], "q": out[2], "r": out[3]}


def far_units(n_units, n_sweep, n_cu, c_begin, nstrip, b):
    a, c = ctypes.c_int64(), ctypes.c_int64()
    load().far_units_c(n_units, n_sweep, n_cu, c_begin, nstrip, b, ctypes.byref(a), ctypes.byref(c))
    return a.value, c.value


def far_sub(n_units, n_sweep, n_cu, c_begin, nstrip, u, u1, d_in):
    out = (ctypes.c_int64 * 4)()
    load().far_sub_c(n_units, n_sweep, n_cu, c_begin, nstrip, u, u1, d_in, out)
    return {"rt": out[0], "c0": out[1], "c_end": out[2], "ns": out[3]}


def far_constants():
    r, c, s = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    load().far_constants(ctypes.byref(r), ctypes.byref(c), ctypes.byref(s))
    return r.value, c.value, s.value
