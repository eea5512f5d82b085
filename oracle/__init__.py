"""fp64 CPU oracle of the fused MoE router (score function + top-k, its
backward, the aux-loss score variant, the load-balancing loss over the aux
scores, decode-shape routing with (expert, token)-sorted expert maps, and
the routed top-k with the shared-expert sigmoid gate folded in).

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
    lib.oracle_select.argtypes = [d, d, i64, i32, i32, i32, i32, u8, d]
    lib.oracle_aux_fwd.argtypes = [d, i64, i32, i32, i32, i32, d, u8, d]
    lib.oracle_aux_bwd.argtypes = [d, d, i64, i32, i32, i32, d]
    q = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_tokens_per_expert.argtypes = [u8, i64, i32, q]
    lib.oracle_aux_loss.argtypes = [d, q, i64, i32, i64, i32, ctypes.c_double, d]
    lib.oracle_aux_loss_bwd.argtypes = [ctypes.c_double, q, i64, i32, i64, i32,
                                        ctypes.c_double, d]
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_route_maps.argtypes = [d, i32, i32, i32, i32, i32, d, i32p, i32p, i32p, i32p, q]
    lib.oracle_topk_shared_gate.argtypes = [d, d, d, i64, i32, i32, i32, i32, i32,
                                            ctypes.c_double, i32, i64, d, i32p]
    for f in (lib.oracle_topk_fwd, lib.oracle_topk_bwd, lib.oracle_select, lib.oracle_aux_fwd,
              lib.oracle_aux_bwd, lib.oracle_tokens_per_expert, lib.oracle_aux_loss,
              lib.oracle_aux_loss_bwd, lib.oracle_route_maps, lib.oracle_topk_shared_gate):
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


def select(key, K, num_groups=0, group_topk=0, gval=None, threads=1, lib=None):
    """The forward's selection step on given keys: returns (routing_map
    [T,E] u8, margin [T] f64) for expert-stage keys ``key`` [T,E] and, with
    groups, group values ``gval`` [T,E] (fp32 values; group scores are
    their fp32 sums)."""
    lib = lib or _load()
    key = _f64(key)
    T, E = key.shape
    gv = None
    if num_groups:
        gv = _f64(gval)
        if gv.shape != key.shape:
            raise OracleError("gval must have the shape of key")
    rmap = np.empty((T, E), np.uint8)
    margin = np.empty((T,), np.float64)
    err = []

    def fn(t0, t1):
        r = lib.oracle_select(
            _p(key[t0:t1], ctypes.c_double),
            None if gv is None else _p(gv[t0:t1], ctypes.c_double), t1 - t0, E, K,
            num_groups, group_topk, _p(rmap[t0:t1], ctypes.c_uint8),
            _p(margin[t0:t1], ctypes.c_double))
        if r != 0:
            err.append(r)

    _run(T, threads, fn)
    if err:
        raise OracleError("oracle_select rejected its arguments")
    return rmap, margin


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


def tokens_per_expert(rmap, lib=None):
    """Column counts of a routing map [T,E] -> int64 [E]."""
    lib = lib or _load()
    m = np.ascontiguousarray(rmap, dtype=np.uint8)
    T, E = m.shape
    out = np.empty((E,), np.int64)
    if lib.oracle_tokens_per_expert(_p(m, ctypes.c_uint8), T, E,
                                    _p(out, ctypes.c_int64)) != 0:
        raise OracleError("oracle_tokens_per_expert rejected its arguments")
    return out


def aux_loss(scores, counts, K, coeff, total_tokens=None, lib=None):
    """Load-balancing loss (float) of scores [T,E] and counts [E]."""
    lib = lib or _load()
    s = _f64(scores)
    c = np.ascontiguousarray(counts, dtype=np.int64)
    T, E = s.shape
    N = T if total_tokens is None else int(total_tokens)
    out = ctypes.c_double()
    if lib.oracle_aux_loss(_p(s, ctypes.c_double), _p(c, ctypes.c_int64), T, E, N, K,
                           float(coeff), ctypes.byref(out)) != 0:
        raise OracleError("oracle_aux_loss rejected its arguments")
    return out.value


def aux_loss_bwd(grad_loss, counts, T, K, coeff, total_tokens=None, lib=None):
    """Gradient [T,E] of the loss with respect to the scores."""
    lib = lib or _load()
    c = np.ascontiguousarray(counts, dtype=np.int64)
    E = c.shape[0]
    N = T if total_tokens is None else int(total_tokens)
    out = np.empty((T, E), np.float64)
    if lib.oracle_aux_loss_bwd(float(grad_loss), _p(c, ctypes.c_int64), T, E, N, K,
                               float(coeff), _p(out, ctypes.c_double)) != 0:
        raise OracleError("oracle_aux_loss_bwd rejected its arguments")
    return out


def route_maps(x, K, score_fn=SOFTMAX, renorm=False, lib=None):
    """Decode routing with expert maps.  Returns a dict: weights [T,K] f64,
    ids [T,K] int32, perm_to_unperm [T*K], unperm_to_perm [T*K],
    perm_expert [T*K] (int32) and expert_offsets [E+1] int64."""
    lib = lib or _load()
    xx = _f64(x)
    T, E = xx.shape
    n = T * K
    out = dict(weights=np.empty((T, K), np.float64), ids=np.empty((T, K), np.int32),
               perm_to_unperm=np.empty((n,), np.int32), unperm_to_perm=np.empty((n,), np.int32),
               perm_expert=np.empty((n,), np.int32), expert_offsets=np.empty((E + 1,), np.int64))
    i32 = ctypes.c_int32
    err = lib.oracle_route_maps(
        _p(xx, ctypes.c_double), T, E, K, score_fn, int(bool(renorm)),
        _p(out["weights"], ctypes.c_double), _p(out["ids"], i32),
        _p(out["perm_to_unperm"], i32), _p(out["unperm_to_perm"], i32),
        _p(out["perm_expert"], i32), _p(out["expert_offsets"], ctypes.c_int64))
    if err:
        raise OracleError("oracle_route_maps rejected its arguments")
    return out


def topk_shared_gate(x, hs, gw, K, renorm=True, scale=1.0, shared_base=None, ld=None,
                     lib=None, threads=1):
    """Routed softmax top-k plus shared-expert gates.  Returns (weights
    [M, ld] f64, ids [M, ld] int32); columns >= K + S are left untouched
    (NaN / -1 here)."""
    lib = lib or _load()
    xx, hh, ww = _f64(x), _f64(hs), _f64(gw)
    M, E = xx.shape
    H = hh.shape[1]
    S = ww.shape[0]
    assert hh.shape[0] == M and ww.shape[1] == H
    base = E if shared_base is None else int(shared_base)
    ld = K + S if ld is None else int(ld)
    w = np.full((M, ld), np.nan)
    ids = np.full((M, ld), -1, np.int32)

    def run(a, b):
        if b <= a:
            return 0
        return lib.oracle_topk_shared_gate(
            _p(xx[a:b], ctypes.c_double), _p(hh[a:b], ctypes.c_double),
            _p(ww, ctypes.c_double), b - a, E, H, K, S, int(bool(renorm)), float(scale),
            base, ld, _p(w[a:b], ctypes.c_double), _p(ids[a:b], ctypes.c_int32))
    if threads > 1 and M > threads:
        step = -(-M // threads)
        with ThreadPoolExecutor(threads) as ex:
            errs = list(ex.map(lambda a: run(a, min(M, a + step)), range(0, M, step)))
    else:
        errs = [run(0, M)]
    if any(errs):
        raise OracleError("oracle_topk_shared_gate rejected its arguments")
    return w, ids
