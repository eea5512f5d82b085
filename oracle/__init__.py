"""fp64 CPU oracle of the fused MoE router (score function + top-k, its
backward, and the aux-loss score variant).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code
with the HIP library and never calls it.

The arithmetic lives in ``router_oracle.c`` (plain C, fp64, one token at a
time); this module only marshals numpy arrays and splits tokens into
contiguous ranges over host threads (the C calls release the GIL).  The
operations follow "[Common] Optimize fused router forward/backward kernels"
(NVIDIA TransformerEngine pull request 3012), sections "Summary",
"Performance" and "Backward kernels"; the C file states each reading taken
where the page is silent.

Parity status: the page prints no worked example, so no output of the
reference itself pins this oracle; the test suite pins it against closed
forms, library routines, brute force and finite differences instead.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

SOFTMAX = 0
SIGMOID = 1

_lib = None


def _load(path=None):
    global _lib
    if path is not None:
        lib = ctypes.CDLL(path)
    else:
        if _lib is not None:
            return _lib
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
    d = ctypes.POINTER(ctypes.c_double)
    u8 = ctypes.POINTER(ctypes.c_uint8)
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.oracle_topk_fwd.argtypes = [d, i64, i32, i32, i32, i32, i32, i32,
                                    ctypes.c_double, d, d, u8, d, d]
    lib.oracle_topk_bwd.argtypes = [d, d, u8, i64, i32, i32, i32, i32,
                                    ctypes.c_double, d]
    lib.oracle_aux_fwd.argtypes = [d, i64, i32, i32, i32, i32, d, u8, d]
    lib.oracle_aux_bwd.argtypes = [d, d, i64, i32, i32, i32, d]
    for f in (lib.oracle_topk_fwd, lib.oracle_topk_bwd, lib.oracle_aux_fwd,
              lib.oracle_aux_bwd):
        f.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a, ct):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ct))


def default_threads():
    return os.cpu_count() or 1


def _run(T, threads, fn):
    """Calls fn(t0, t1) over contiguous token ranges on ``threads`` threads."""
    threads = max(1, min(int(threads or 1), T if T > 0 else 1))
    if threads == 1 or T < 2:
        fn(0, T)
        return
    step = (T + threads - 1) // threads
    ranges = [(a, min(T, a + step)) for a in range(0, T, step)]
    with ThreadPoolExecutor(len(ranges)) as ex:
        list(ex.map(lambda r: fn(*r), ranges))


class OracleError(ValueError):
    pass


def topk_fwd(x, K, score_fn=SOFTMAX, renorm=False, num_groups=0,
             group_topk=0, scaling_factor=1.0, bias=None, threads=1,
             lib=None):
    """Returns (probs [T,E] f64, routing_map [T,E] u8, intermediate [T,E]
    f64, margin [T] f64) for logits x [T,E]."""
    lib = lib or _load()
    x = _f64(x)
    T, E = x.shape
    b = None if bias is None else _f64(bias)
    probs = np.empty((T, E), np.float64)
    rmap = np.empty((T, E), np.uint8)
    inter = np.empty((T, E), np.float64)
    margin = np.empty((T,), np.float64)
    err = []

    def fn(t0, t1):
        r = lib.oracle_topk_fwd(
            _p(x[t0:t1], ctypes.c_double), t1 - t0, E, K, score_fn,
            int(bool(renorm)), num_groups, group_topk, float(scaling_factor),
            _p(b, ctypes.c_double), _p(probs[t0:t1], ctypes.c_double),
            _p(rmap[t0:t1], ctypes.c_uint8), _p(inter[t0:t1], ctypes.c_double),
            _p(margin[t0:t1], ctypes.c_double))
        if r != 0:
            err.append(r)

    _run(T, threads, fn)
    if err:
        raise OracleError("oracle_topk_fwd rejected its arguments")
    return probs, rmap, inter, margin


def topk_bwd(g, s, m, K, score_fn=SOFTMAX, renorm=False, scaling_factor=1.0,
             threads=1, lib=None):
    """Returns grad_logits [T,E] f64 from grad_probs g, intermediate s and
    routing_map m (all [T,E])."""
    lib = lib or _load()
    g, s = _f64(g), _f64(s)
    m = np.ascontiguousarray(m, dtype=np.uint8)
    T, E = g.shape
    dx = np.empty((T, E), np.float64)
    err = []

    def fn(t0, t1):
        r = lib.oracle_topk_bwd(
            _p(g[t0:t1], ctypes.c_double), _p(s[t0:t1], ctypes.c_double),
            _p(m[t0:t1], ctypes.c_uint8), t1 - t0, E, K, score_fn,
            int(bool(renorm)), float(scaling_factor),
            _p(dx[t0:t1], ctypes.c_double))
        if r != 0:
            err.append(r)

    _run(T, threads, fn)
    if err:
        raise OracleError("oracle_topk_bwd rejected its arguments")
    return dx


def aux_fwd(x, K, score_fn=SOFTMAX, renorm=True, threads=1, lib=None):
    """Returns (scores [T,E] f64, routing_map [T,E] u8, intermediate [T,E]
    f64) for logits x [T,E]."""
    lib = lib or _load()
    x = _f64(x)
    T, E = x.shape
    scores = np.empty((T, E), np.float64)
    rmap = np.empty((T, E), np.uint8)
    inter = np.empty((T, E), np.float64)
    err = []

    def fn(t0, t1):
        r = lib.oracle_aux_fwd(
            _p(x[t0:t1], ctypes.c_double), t1 - t0, E, K, score_fn,
            int(bool(renorm)), _p(scores[t0:t1], ctypes.c_double),
            _p(rmap[t0:t1], ctypes.c_uint8), _p(inter[t0:t1], ctypes.c_double))
        if r != 0:
            err.append(r)

    _run(T, threads, fn)
    if err:
        raise OracleError("oracle_aux_fwd rejected its arguments")
    return scores, rmap, inter


def aux_bwd(g, s, score_fn=SOFTMAX, renorm=True, threads=1, lib=None):
    """Returns grad_logits [T,E] f64 from grad_scores g and intermediate s."""
    lib = lib or _load()
    g, s = _f64(g), _f64(s)
    T, E = g.shape
    dx = np.empty((T, E), np.float64)
    err = []

    def fn(t0, t1):
        r = lib.oracle_aux_bwd(
            _p(g[t0:t1], ctypes.c_double), _p(s[t0:t1], ctypes.c_double),
            t1 - t0, E, score_fn, int(bool(renorm)),
            _p(dx[t0:t1], ctypes.c_double))
        if r != 0:
            err.append(r)

    _run(T, threads, fn)
    if err:
        raise OracleError("oracle_aux_bwd rejected its arguments")
    return dx
