"""Pins of the fp64 router oracle against facts that do not come from the
oracle itself: hand-derived closed forms (tests/golden), library routines
(scipy's softmax and logistic sigmoid), exhaustive brute force over all
subsets on tiny inputs, central finite differences of the forward, and
invariants of the mathematics (shift invariance, linearity, masking).

Every pin takes the loaded oracle library, so the mutation test can run the
same pins against deliberately broken copies of the oracle.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
SCORE = {"softmax": oracle.SOFTMAX, "sigmoid": oracle.SIGMOID}


# --------------------------------------------------------------- helpers

def close(a, b, rtol=1e-12, atol=1e-14, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    ok = np.abs(a - b) <= atol + rtol * np.abs(b)
    assert ok.all(), f"{what}: max err {np.max(np.abs(a - b))}\n{a}\n{b}"


def defining_property(key, sel, allowed=None):
    """True iff every selected j beats every unselected allowed i: larger
    key, or equal key and lower index."""
    E = len(key)
    allowed = np.ones(E, bool) if allowed is None else allowed
    for j in range(E):
        if not sel[j]:
            continue
        for i in range(E):
            if sel[i] or not allowed[i]:
                continue
            if not (key[j] > key[i] or (key[j] == key[i] and j < i)):
                return False
    return True


def brute_select(key, K, allowed=None):
    """The unique K-subset of allowed indices that satisfies the defining
    property, found by enumerating every subset."""
    E = len(key)
    allowed = np.ones(E, bool) if allowed is None else allowed
    idx = [j for j in range(E) if allowed[j]]
    found = []
    for sub in itertools.combinations(idx, K):
        sel = np.zeros(E, bool)
        sel[list(sub)] = True
        if defining_property(key, sel, allowed):
            found.append(sel)
    assert len(found) == 1, f"{len(found)} subsets satisfy the property"
    return found[0]


def f32_sigmoid(x):
    return scipy.special.expit(np.asarray(x, np.float64)).astype(np.float32)


def biased_key(x, b):
    """Selection key with a bias: s rounded to fp32, plus the fp32 bias, in
    fp32 arithmetic."""
    return (f32_sigmoid(x) + np.asarray(b, np.float32)).astype(np.float64)


def group_values(x, score_fn, b):
    s = (scipy.special.softmax(x) if score_fn == oracle.SOFTMAX
         else scipy.special.expit(x)).astype(np.float32)
    if b is not None:
        s = (s + np.asarray(b, np.float32)).astype(np.float32)
    return s


def brute_group_select(gv, G, Kg, q):
    """Kept groups: group score = best fp32 sum over every q-subset of the
    group (largest member first); then the unique Kg-subset of groups with
    the defining property."""
    per = len(gv) // G
    h = np.zeros(G)
    for g in range(G):
        best = -np.inf
        for sub in itertools.combinations(range(per), q):
            vals = sorted((gv[g * per + i] for i in sub), reverse=True)
            acc = np.float32(0)
            for v in vals:
                acc = np.float32(acc + np.float32(v))
            best = max(best, float(acc))
        h[g] = best
    return brute_select(h, Kg)


def parse_golden(path):
    cases, cur = [], None
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = [p.strip() for p in line.split(":", 1)]
            if k == "case":
                cur = {"case": v}
                cases.append(cur)
                continue
            if k in ("op", "score"):
                cur[k] = v
            else:
                vals = [float(Fraction(t)) for t in v.split()]
                cur[k] = vals if len(vals) > 1 or k in (
                    "w", "s", "m", "g", "map", "probs", "inter", "scores",
                    "dx", "bias", "counts", "dscore", "ids", "weights", "perm_to_unperm",
                    "unperm_to_perm", "perm_expert", "expert_offsets", "hs_ln",
                    "gw") else vals[0]
    return cases


# ------------------------------------------------------------------ pins

def pin_golden(lib):
    """Hand-derived closed forms under tests/golden."""
    n = 0
    for fn in sorted(os.listdir(GOLDEN)):
        if not fn.endswith(".txt") or fn == "README.txt":
            continue
        for c in parse_golden(os.path.join(GOLDEN, fn)):
            what = f"{fn}:{c['case']}"
            if c["op"] == "aux_loss":
                golden_aux_loss(lib, c, what)
                n += 1
                continue
            if c["op"] == "route_maps":
                golden_route_maps(lib, c, what)
                n += 1
                continue
            if c["op"] == "topk_shared_gate":
                golden_shared_gate(lib, c, what)
                n += 1
                continue
            sf = SCORE[c["score"]]
            if c["op"] == "topk_fwd":
                x = np.log(np.array(c["w"]))[None]
                b = None if "bias" not in c else np.array(c["bias"])
                p, m, i, _ = oracle.topk_fwd(
                    x, int(c["K"]), sf, bool(c["renorm"]),
                    int(c.get("groups", 0)), int(c.get("group_topk", 0)),
                    c["c"], b, lib=lib)
                assert (m[0] == np.array(c["map"])).all(), (what, m)
                close(p[0], c["probs"], what=what + " probs")
                close(i[0], c["inter"], what=what + " inter")
            elif c["op"] == "aux_fwd":
                x = np.log(np.array(c["w"]))[None]
                sc, m, i = oracle.aux_fwd(x, int(c["K"]), sf,
                                          bool(c["renorm"]), lib=lib)
                assert (m[0] == np.array(c["map"])).all(), (what, m)
                close(sc[0], c["scores"], what=what + " scores")
                close(i[0], c["inter"], what=what + " inter")
            elif c["op"] == "topk_bwd":
                dx = oracle.topk_bwd(
                    np.array(c["g"])[None], np.array(c["s"])[None],
                    np.array(c["m"], np.uint8)[None], int(c["K"]), sf,
                    bool(c["renorm"]), c["c"], lib=lib)
                close(dx[0], c["dx"], what=what)
            elif c["op"] == "aux_bwd":
                dx = oracle.aux_bwd(np.array(c["g"])[None],
                                    np.array(c["s"])[None], sf,
                                    bool(c["renorm"]), lib=lib)
                close(dx[0], c["dx"], what=what)
            else:
                raise AssertionError(what)
            n += 1
    assert n == 26, n


def golden_shared_gate(lib, c, what):
    E, H, K, S = int(c["E"]), int(c["H"]), int(c["K"]), int(c["S"])
    x = np.log(np.array(c["w"])).reshape(-1, E)
    hs = np.log(np.array(c["hs_ln"], dtype=np.float64).reshape(-1, H))
    gw = np.array(c["gw"], dtype=np.float64).reshape(S, H)
    w, ids = oracle.topk_shared_gate(x, hs, gw, K, bool(c["renorm"]), c["scale"],
                                     int(c["base"]), lib=lib)
    assert (ids.ravel() == np.array(c["ids"])).all(), (what, ids)
    close(w.ravel(), c["weights"], what=what + " weights")


def golden_route_maps(lib, c, what):
    T, E, K = int(c["T"]), int(c["E"]), int(c["K"])
    x = np.log(np.array(c["w"])).reshape(T, E)
    r = oracle.route_maps(x, K, SCORE[c["score"]], bool(c["renorm"]), lib=lib)
    for f in ("ids", "perm_to_unperm", "unperm_to_perm", "perm_expert", "expert_offsets"):
        assert (r[f].ravel() == np.array(c[f])).all(), (what, f, r[f])
    close(r["weights"].ravel(), c["weights"], what=what + " weights")


def golden_aux_loss(lib, c, what):
    E = int(c["E"])
    sc = np.array(c["scores"]).reshape(-1, E)
    if "map" in c:
        m = np.array(c["map"], np.uint8).reshape(-1, E)
        cnt = oracle.tokens_per_expert(m, lib=lib)
        assert (cnt == np.array(c["counts"])).all(), (what, cnt)
    cnt = np.array(c["counts"], np.int64)
    K, coeff, N = int(c["K"]), c["coeff"], int(c["N"])
    close(oracle.aux_loss(sc, cnt, K, coeff, N, lib=lib), c["loss"], what=what + " loss")
    d = oracle.aux_loss_bwd(c["grad_loss"], cnt, sc.shape[0], K, coeff, N, lib=lib)
    close(d.ravel(), c["dscore"], what=what + " dscore")


def pin_score_library(lib):
    """Scores equal scipy's softmax / logistic sigmoid; softmax sums to 1
    and is unchanged (with its selection) by a row shift of +1000."""
    rng = np.random.default_rng(11)
    x = rng.normal(0, 3, (6, 37))
    _, m, i, _ = oracle.topk_fwd(x, 5, oracle.SOFTMAX, lib=lib)
    close(i, scipy.special.softmax(x, axis=1), rtol=1e-13, atol=1e-16,
          what="softmax")
    close(i.sum(1), np.ones(6), rtol=1e-13, what="softmax sum")
    _, m2, i2, _ = oracle.topk_fwd(x + 1000.0, 5, oracle.SOFTMAX, lib=lib)
    assert (m2 == m).all()
    close(i2, i, rtol=1e-9, atol=1e-15, what="softmax shift")
    _, _, i3, _ = oracle.topk_fwd(x, 5, oracle.SIGMOID, lib=lib)
    close(i3, scipy.special.expit(x), rtol=1e-13, what="sigmoid")
    _, _, i4, _ = oracle.topk_fwd(-x, 5, oracle.SIGMOID, lib=lib)
    close(i4, 1.0 - i3, rtol=1e-12, atol=1e-15, what="sigmoid symmetry")


def pin_topk_bruteforce(lib):
    """Maps equal the unique subset with the defining property, by
    enumeration, on tiny rows full of ties; several tokens at once."""
    rng = np.random.default_rng(12)
    for E in (1, 2, 5, 9):
        for K in range(1, min(E, 4) + 1):
            x = rng.integers(-2, 3, (5, E)).astype(np.float64)
            for sf in (oracle.SOFTMAX, oracle.SIGMOID):
                _, m, _, _ = oracle.topk_fwd(x, K, sf, lib=lib)
                for t in range(5):
                    assert (m[t] == brute_select(x[t], K)).all(), (E, K, t)
            _, m, _ = oracle.aux_fwd(x, K, oracle.SOFTMAX, lib=lib)
            for t in range(5):
                assert (m[t] == brute_select(x[t], K)).all(), (E, K, t)
    # biased sigmoid: selection on the fp32 key s + b
    x = rng.normal(0, 1, (6, 8))
    b = rng.choice([-0.1, 0.0, 0.05, 0.1], 8)
    b = b.astype(np.float32).astype(np.float64)
    for K in (1, 3):
        _, m, _, _ = oracle.topk_fwd(x, K, oracle.SIGMOID, True, bias=b,
                                     lib=lib)
        for t in range(6):
            assert (m[t] == brute_select(biased_key(x[t], b), K)).all()


def pin_groups_bruteforce(lib):
    """Group-limited maps equal brute force over every subset of groups
    and of experts; one group (or every group kept) is plain top-K."""
    rng = np.random.default_rng(13)
    for (E, G, Kg, K) in ((8, 4, 2, 4), (12, 6, 3, 3), (12, 4, 2, 2),
                          (6, 3, 1, 2), (12, 6, 2, 4)):
        q = K // Kg
        for sf in (oracle.SIGMOID, oracle.SOFTMAX):
            x = rng.integers(-2, 3, (4, E)).astype(np.float64) * 0.5
            b = None
            if sf == oracle.SIGMOID:
                b = rng.choice([-0.25, 0.0, 0.125], E)
            _, m, _, _ = oracle.topk_fwd(x, K, sf, True, G, Kg, 1.0, b,
                                         lib=lib)
            for t in range(4):
                gv = group_values(x[t], sf, b)
                kept = brute_group_select(gv.astype(np.float64), G, Kg, q)
                allowed = np.repeat(kept, E // G)
                key = biased_key(x[t], b) if b is not None else x[t]
                want = brute_select(key, K, allowed)
                assert (m[t] == want).all(), (E, G, Kg, K, sf, t, m[t], want)
    x = rng.normal(0, 1, (5, 12))
    _, m0, _, _ = oracle.topk_fwd(x, 4, oracle.SIGMOID, lib=lib)
    _, m1, _, _ = oracle.topk_fwd(x, 4, oracle.SIGMOID, False, 1, 1, lib=lib)
    _, m2, _, _ = oracle.topk_fwd(x, 4, oracle.SIGMOID, False, 4, 4, lib=lib)
    assert (m0 == m1).all() and (m0 == m2).all()


def pin_select_bruteforce(lib):
    """The selection step on given keys and group values equals brute force
    over every subset of groups and of experts (tiny tie-heavy rows, keys
    independent of the group values), and, fed the forward's own keys, it
    reproduces the forward's map and margin."""
    rng = np.random.default_rng(17)
    for (E, G, Kg, K) in ((6, 0, 0, 1), (9, 0, 0, 3), (8, 4, 2, 4), (12, 6, 3, 3),
                          (12, 4, 2, 2), (6, 3, 1, 2), (12, 6, 2, 4)):
        key = rng.integers(-2, 3, (5, E)).astype(np.float64)
        gv = (rng.integers(0, 4, (5, E)) * 0.25).astype(np.float32).astype(np.float64)
        m, _ = oracle.select(key, K, G, Kg, gv if G else None, lib=lib)
        for t in range(5):
            allowed = None
            if G:
                kept = brute_group_select(gv[t], G, Kg, K // Kg)
                allowed = np.repeat(kept, E // G)
            assert (m[t] == brute_select(key[t], K, allowed)).all(), (E, G, Kg, K, t)
    x = rng.normal(0, 1, (7, 24))
    b = rng.uniform(-0.1, 0.1, 24).astype(np.float32).astype(np.float64)
    _, m0, _, mg0 = oracle.topk_fwd(x, 6, oracle.SIGMOID, True, 4, 2, 1.0, b, lib=lib)
    gv = np.stack([group_values(r, oracle.SIGMOID, b) for r in x]).astype(np.float64)
    m1, mg1 = oracle.select(gv, 6, 4, 2, gv, lib=lib)
    assert (m0 == m1).all()
    close(mg1, mg0, rtol=0, atol=0, what="select margin")


def pin_renorm_identities(lib):
    """Renormalised probs sum to c; softmax renorm is scipy's softmax over
    the selected logits; with K = E the topk scores equal the aux scores."""
    rng = np.random.default_rng(14)
    x = rng.normal(0, 2, (4, 10))
    for sf in (oracle.SOFTMAX, oracle.SIGMOID):
        p, m, _, _ = oracle.topk_fwd(x, 3, sf, True, scaling_factor=1.75,
                                     lib=lib)
        close(p.sum(1), np.full(4, 1.75), rtol=1e-13, what="renorm sum")
    p, m, _, _ = oracle.topk_fwd(x, 3, oracle.SOFTMAX, True, lib=lib)
    for t in range(4):
        sel = m[t].astype(bool)
        close(p[t][sel], scipy.special.softmax(x[t][sel]), rtol=1e-13,
              what="softmax over selected")
    p, _, _, _ = oracle.topk_fwd(x, 10, oracle.SIGMOID, True, lib=lib)
    a, am, _ = oracle.aux_fwd(x, 10, oracle.SIGMOID, True, lib=lib)
    close(p, a, rtol=1e-13, what="sigmoid renorm K=E vs aux")
    assert am.all()
    p, _, _, _ = oracle.topk_fwd(x, 10, oracle.SOFTMAX, False, lib=lib)
    a, _, _ = oracle.aux_fwd(x, 10, oracle.SOFTMAX, True, lib=lib)
    close(p, a, rtol=1e-13, what="softmax K=E vs aux")
    a, _, i = oracle.aux_fwd(x, 3, oracle.SIGMOID, False, lib=lib)
    close(a, scipy.special.expit(x), rtol=1e-13, what="aux raw sigmoid")
    close(i, scipy.special.expit(x), rtol=1e-13, what="aux sigmoid inter")


def pin_scale_linearity(lib):
    """probs and gradients scale linearly with the scaling factor."""
    rng = np.random.default_rng(15)
    x = rng.normal(0, 1, (3, 9))
    g = rng.normal(0, 1, (3, 9))
    for sf in (oracle.SOFTMAX, oracle.SIGMOID):
        for rn in (False, True):
            p1, m, s, _ = oracle.topk_fwd(x, 3, sf, rn, scaling_factor=1.0,
                                          lib=lib)
            p3, _, _, _ = oracle.topk_fwd(x, 3, sf, rn, scaling_factor=3.0,
                                          lib=lib)
            close(p3, 3 * p1, rtol=1e-14, what="probs linear in c")
            d1 = oracle.topk_bwd(g, s, m, 3, sf, rn, 1.0, lib=lib)
            d3 = oracle.topk_bwd(g, s, m, 3, sf, rn, 3.0, lib=lib)
            close(d3, 3 * d1, rtol=1e-14, atol=1e-300, what="grad linear")


def _fd_check(lib, x, g, K, sf, rn, G, Kg, c, b, aux=False, h=1e-5):
    if aux:
        _, m, s = oracle.aux_fwd(x, K, sf, rn, lib=lib)
        dx = oracle.aux_bwd(g, s, sf, rn, lib=lib)
    else:
        _, m, s, _ = oracle.topk_fwd(x, K, sf, rn, G, Kg, c, b, lib=lib)
        dx = oracle.topk_bwd(g, s, m, K, sf, rn, c, lib=lib)
    T, E = x.shape
    checked = 0
    for t in range(T):
        for k in range(E):
            xp, xm = x[t:t + 1].copy(), x[t:t + 1].copy()
            xp[0, k] += h
            xm[0, k] -= h
            if aux:
                pp, mp, _ = oracle.aux_fwd(xp, K, sf, rn, lib=lib)
                pm, mm, _ = oracle.aux_fwd(xm, K, sf, rn, lib=lib)
            else:
                pp, mp, _, _ = oracle.topk_fwd(xp, K, sf, rn, G, Kg, c, b,
                                               lib=lib)
                pm, mm, _, _ = oracle.topk_fwd(xm, K, sf, rn, G, Kg, c, b,
                                               lib=lib)
            if not aux and ((mp[0] != m[t]).any() or (mm[0] != m[t]).any()):
                continue
            fd = (np.dot(g[t], pp[0]) - np.dot(g[t], pm[0])) / (2 * h)
            assert abs(fd - dx[t, k]) <= 1e-7 + 1e-6 * abs(dx[t, k]), (
                sf, rn, G, b is not None, aux, t, k, fd, dx[t, k])
            checked += 1
    assert checked >= T * E // 2, checked


def pin_backward_fd(lib):
    """topk backward equals central finite differences of the forward for
    every score function x renorm x bias x groups combination."""
    rng = np.random.default_rng(16)
    for sf in (oracle.SOFTMAX, oracle.SIGMOID):
        for rn in (False, True):
            for grouped in (False, True):
                for biased in ((False, True) if sf == oracle.SIGMOID
                               else (False,)):
                    E, K = 12, 4
                    G, Kg = (4, 2) if grouped else (0, 0)
                    x = rng.normal(0, 1.5, (3, E))
                    g = rng.normal(0, 1, (3, E))
                    b = rng.uniform(-0.1, 0.1, E) if biased else None
                    _fd_check(lib, x, g, K, sf, rn, G, Kg, 1.7, b)
    x = rng.normal(0, 1, (2, 7))
    g = rng.normal(0, 1, (2, 7))
    _fd_check(lib, x, g, 1, oracle.SIGMOID, True, 0, 0, 1.3, None)


def pin_aux_backward_fd(lib):
    """aux backward equals finite differences of the aux scores."""
    rng = np.random.default_rng(17)
    for sf, rn in ((oracle.SOFTMAX, True), (oracle.SIGMOID, True),
                   (oracle.SIGMOID, False)):
        x = rng.normal(0, 1.5, (3, 11))
        g = rng.normal(0, 1, (3, 11))
        _fd_check(lib, x, g, 3, sf, rn, 0, 0, 1.0, None, aux=True)


def pin_backward_invariants(lib):
    """Softmax gradients sum to zero over a row (shift invariance); the
    backward is linear in g; bwd(g) = bwd(g*m); off-map gradients vanish
    for sigmoid and for softmax with renorm."""
    rng = np.random.default_rng(18)
    x = rng.normal(0, 1, (5, 16))
    g1 = rng.normal(0, 1, (5, 16))
    g2 = rng.normal(0, 1, (5, 16))
    for sf in (oracle.SOFTMAX, oracle.SIGMOID):
        for rn in (False, True):
            _, m, s, _ = oracle.topk_fwd(x, 4, sf, rn, lib=lib)
            d1 = oracle.topk_bwd(g1, s, m, 4, sf, rn, 1.0, lib=lib)
            d2 = oracle.topk_bwd(g2, s, m, 4, sf, rn, 1.0, lib=lib)
            d12 = oracle.topk_bwd(2 * g1 - g2, s, m, 4, sf, rn, 1.0, lib=lib)
            close(d12, 2 * d1 - d2, rtol=1e-12, atol=1e-14, what="linear g")
            dm = oracle.topk_bwd(g1 * m, s, m, 4, sf, rn, 1.0, lib=lib)
            close(dm, d1, rtol=1e-14, atol=1e-300, what="bwd(g*m)")
            if sf == oracle.SOFTMAX:
                close(d1.sum(1), np.zeros(5), atol=1e-14, what="sum dx")
            if sf == oracle.SIGMOID or rn:
                assert (d1[m == 0] == 0).all()
    _, _, s = oracle.aux_fwd(x, 4, oracle.SOFTMAX, True, lib=lib)
    d = oracle.aux_bwd(g1, s, oracle.SOFTMAX, True, lib=lib)
    close(d.sum(1), np.zeros(5), atol=1e-14, what="aux sum dx")


def pin_rows_independent(lib):
    """A batch gives the same outputs as each row on its own."""
    rng = np.random.default_rng(19)
    x = rng.normal(0, 1, (4, 10))
    g = rng.normal(0, 1, (4, 10))
    b = rng.uniform(-0.1, 0.1, 10)
    P, M, S, _ = oracle.topk_fwd(x, 4, oracle.SIGMOID, True, 5, 2, 2.0, b,
                                 lib=lib)
    D = oracle.topk_bwd(g, S, M, 4, oracle.SIGMOID, True, 2.0, lib=lib)
    A, AM, AS = oracle.aux_fwd(x, 3, oracle.SIGMOID, True, lib=lib)
    AD = oracle.aux_bwd(g, AS, oracle.SIGMOID, True, lib=lib)
    for t in range(4):
        p, m, s, _ = oracle.topk_fwd(x[t:t + 1], 4, oracle.SIGMOID, True, 5,
                                     2, 2.0, b, lib=lib)
        assert (m == M[t]).all()
        close(p, P[t:t + 1], rtol=0, atol=0)
        close(oracle.topk_bwd(g[t:t + 1], s, m, 4, oracle.SIGMOID, True,
                              2.0, lib=lib), D[t:t + 1], rtol=0, atol=0)
        a, am, as_ = oracle.aux_fwd(x[t:t + 1], 3, oracle.SIGMOID, True,
                                    lib=lib)
        close(a, A[t:t + 1], rtol=0, atol=0)
        close(oracle.aux_bwd(g[t:t + 1], as_, oracle.SIGMOID, True, lib=lib),
              AD[t:t + 1], rtol=0, atol=0)


def pin_margin(lib):
    """The reported margin is the gap between the last kept and the first
    dropped key (logits 3, 1.5, 1, 0 with K = 2: gap 0.5)."""
    x = np.array([[1.0, 3.0, 0.0, 1.5]])
    _, _, _, mg = oracle.topk_fwd(x, 2, oracle.SOFTMAX, lib=lib)
    close(mg, [0.5], what="margin")
    _, _, _, mg = oracle.topk_fwd(x, 4, oracle.SOFTMAX, lib=lib)
    assert np.isinf(mg[0])


def pin_tokens_per_expert(lib):
    """Column counts of random maps equal numpy's column sums, including a
    map with empty columns and one with no rows."""
    rng = np.random.default_rng(11)
    for T, E, p in ((1, 1, 0.5), (7, 5, 0.3), (33, 64, 0.05), (64, 9, 0.9)):
        m = (rng.random((T, E)) < p).astype(np.uint8)
        m[:, 0] = 0
        assert (oracle.tokens_per_expert(m, lib=lib) == m.sum(0)).all(), (T, E)
    assert (oracle.tokens_per_expert(np.zeros((0, 6), np.uint8), lib=lib) == 0).all()


def pin_aux_loss_closed_forms(lib):
    """Balanced routing (every score 1/E, every count N K / E) gives exactly
    coeff; one expert taking everything gives coeff * E; the loss is linear
    in the scores, scales as 1/N^2 at fixed sums, and is invariant to the
    order of the tokens and to a relabelling of the experts."""
    rng = np.random.default_rng(12)
    for N, E, K, coeff in ((8, 4, 2, 0.01), (12, 6, 3, 1.0), (64, 16, 4, 1e-3)):
        sc = np.full((N, E), 1.0 / E)
        cnt = np.full(E, N * K // E, np.int64)
        close(oracle.aux_loss(sc, cnt, K, coeff, lib=lib), coeff, what="balanced")
        sc = np.zeros((N, E))
        sc[:, 1] = 1.0
        cnt = np.zeros(E, np.int64)
        cnt[1] = N * K
        close(oracle.aux_loss(sc, cnt, K, coeff, lib=lib), coeff * E,
              what="collapse")
    T, E, K = 9, 7, 3
    a, b = rng.random((T, E)), rng.random((T, E))
    cnt = rng.integers(0, 20, E)
    la = oracle.aux_loss(a, cnt, K, 0.3, 40, lib=lib)
    lb = oracle.aux_loss(b, cnt, K, 0.3, 40, lib=lib)
    close(oracle.aux_loss(2 * a - b, cnt, K, 0.3, 40, lib=lib), 2 * la - lb, what="linear")
    close(oracle.aux_loss(a, cnt, K, 0.3, 80, lib=lib), la / 4, what="1/N^2")
    perm_t, perm_e = rng.permutation(T), rng.permutation(E)
    close(oracle.aux_loss(a[perm_t][:, perm_e], cnt[perm_e], K, 0.3, 40, lib=lib), la,
          what="relabel")
    # brute force: the double sum over tokens and experts, term by term
    want = sum(a[t, i] * cnt[i] for t in range(T) for i in range(E)) * 0.3 * E / (40 * 40 * K)
    close(la, want, what="double sum")


def pin_aux_loss_fd(lib):
    """The gradient of the loss equals its central finite difference in
    every score (the loss is linear, so the difference is exact up to
    rounding), scaled by grad_loss."""
    rng = np.random.default_rng(13)
    T, E, K, coeff, N = 5, 6, 2, 0.05, 12
    sc = rng.random((T, E))
    cnt = rng.integers(0, 9, E)
    d = oracle.aux_loss_bwd(-1.5, cnt, T, K, coeff, N, lib=lib)
    h = 1e-3
    fd = np.empty_like(sc)
    for t in range(T):
        for i in range(E):
            up, dn = sc.copy(), sc.copy()
            up[t, i] += h
            dn[t, i] -= h
            fd[t, i] = (oracle.aux_loss(up, cnt, K, coeff, N, lib=lib) -
                        oracle.aux_loss(dn, cnt, K, coeff, N, lib=lib)) / (2 * h)
    close(d, -1.5 * fd, rtol=1e-9, atol=1e-13, what="aux loss fd")


def check_maps_structure(r, T, E, K, what=""):
    """The maps are a permutation and its inverse, sorted by (expert,
    token), with offsets equal to the cumulative expert histogram."""
    n = T * K
    p2u, u2p, pe, off = (r["perm_to_unperm"], r["unperm_to_perm"], r["perm_expert"],
                         r["expert_offsets"])
    assert sorted(p2u.tolist()) == list(range(n)), what
    assert (u2p[p2u] == np.arange(n)).all(), what
    tok = p2u % T if T else p2u
    key = pe.astype(np.int64) * max(T, 1) + tok
    assert (np.diff(key) > 0).all(), what
    ids = r["ids"]
    assert (pe == ids.T.ravel()[p2u]).all(), what
    cnt = np.bincount(ids.ravel(), minlength=E)
    assert (off == np.concatenate([[0], np.cumsum(cnt)])).all(), what


def pin_route_maps_bruteforce(lib):
    """Selection against numpy's lexsort (logit descending, index
    ascending), weights against scipy's softmax / logistic sigmoid, maps
    against a lexsort of the pairs by (expert, token) and a bincount, on
    random rows with heavy ties."""
    rng = np.random.default_rng(21)
    for T, E, K, sf, rn in ((1, 8, 3, oracle.SOFTMAX, False), (4, 512, 10, oracle.SOFTMAX, True),
                            (3, 40, 6, oracle.SIGMOID, True), (4, 16, 16, oracle.SOFTMAX, True),
                            (2, 7, 1, oracle.SIGMOID, True), (4, 64, 8, oracle.SIGMOID, False)):
        x = rng.integers(-3, 4, (T, E)).astype(np.float64)   # many ties
        r = oracle.route_maps(x, K, sf, rn, lib=lib)
        s = scipy.special.softmax(x, axis=1) if sf == oracle.SOFTMAX else scipy.special.expit(x)
        ids = np.stack([np.lexsort((np.arange(E), -x[t]))[:K] for t in range(T)])
        assert (r["ids"] == ids).all(), (T, E, K)
        w = np.take_along_axis(s, ids, 1)
        if rn and (sf == oracle.SOFTMAX or K > 1):
            w = w / w.sum(1, keepdims=True)
        close(r["weights"], w, what="route weights")
        exp = ids.T.ravel()                    # expert of unpermuted index u = t + k*T
        tok = np.tile(np.arange(T), K)
        order = np.lexsort((tok, exp))
        assert (r["perm_to_unperm"] == order).all()
        assert (r["perm_expert"] == exp[order]).all()
        check_maps_structure(r, T, E, K)


def pin_route_maps_vs_topk(lib):
    """The selected set and weights equal the top-k forward's routing map
    and probs (same scores, renorm rule, no scaling)."""
    rng = np.random.default_rng(22)
    for sf, rn in ((oracle.SOFTMAX, False), (oracle.SOFTMAX, True), (oracle.SIGMOID, True)):
        x = rng.normal(0, 2, (4, 96))
        r = oracle.route_maps(x, 9, sf, rn, lib=lib)
        P, M, _, _ = oracle.topk_fwd(x, 9, sf, rn, lib=lib)
        for t in range(4):
            assert sorted(r["ids"][t].tolist()) == np.nonzero(M[t])[0].tolist()
            close(r["weights"][t], P[t, r["ids"][t]], what="route vs topk")
        assert (np.diff(np.take_along_axis(x, r["ids"].astype(np.int64), 1), axis=1) <= 0).all()


def pin_shared_gate_library(lib):
    """Routed part against numpy lexsort and scipy softmax, gates against
    scipy's expit of numpy's dot, on the page's test axes (S in {1, 2, 8},
    renorm on/off, scale 0.5, M = 1 and 65), with a wider output row whose
    extra columns stay untouched."""
    rng = np.random.default_rng(31)
    for M, E, H, K, S, rn, sc in ((1, 512, 64, 10, 1, True, 1.0), (65, 256, 48, 8, 2, False, 0.5),
                                  (9, 64, 40, 6, 8, True, 0.5), (4, 20, 7, 20, 3, True, 2.0)):
        x = rng.integers(-3, 4, (M, E)).astype(np.float64)      # ties
        hs = rng.normal(0, 1, (M, H))
        gw = rng.normal(0, 0.2, (S, H))
        ld = K + S + 3
        w, ids = oracle.topk_shared_gate(x, hs, gw, K, rn, sc, 1000, ld, lib=lib)
        sm = scipy.special.softmax(x, axis=1)
        top = np.stack([np.lexsort((np.arange(E), -x[m]))[:K] for m in range(M)])
        assert (ids[:, :K] == top).all()
        wr = np.take_along_axis(sm, top, 1)
        if rn:
            wr = wr / wr.sum(1, keepdims=True)
        close(w[:, :K], wr, what="shared-gate routed")
        close(w[:, K:K + S], sc * scipy.special.expit(hs @ gw.T), rtol=1e-12, atol=1e-15,
              what="shared gates")
        assert (ids[:, K:K + S] == 1000 + np.arange(S)).all()
        assert np.isnan(w[:, K + S:]).all() and (ids[:, K + S:] == -1).all()


def pin_shared_gate_invariants(lib):
    """The routed columns equal the decode routing oracle's softmax slots;
    the gates scale linearly with `scale`, ignore the gating logits, and
    swap with the gate-weight rows."""
    rng = np.random.default_rng(32)
    x = rng.normal(0, 2, (6, 128))
    hs = rng.normal(0, 1, (6, 33))
    gw = rng.normal(0, 0.3, (4, 33))
    w, ids = oracle.topk_shared_gate(x, hs, gw, 7, True, 1.0, 128, lib=lib)
    r = oracle.route_maps(x, 7, oracle.SOFTMAX, True, lib=lib)
    assert (ids[:, :7] == r["ids"]).all()
    close(w[:, :7], r["weights"], what="routed vs route maps")
    w2, _ = oracle.topk_shared_gate(-x, hs, gw, 7, True, 3.0, 128, lib=lib)
    close(w2[:, 7:], 3.0 * w[:, 7:], what="scale / gating independence")
    w3, _ = oracle.topk_shared_gate(x, hs, gw[::-1].copy(), 7, True, 1.0, 128, lib=lib)
    close(w3[:, 7:], w[:, 7:][:, ::-1], what="gate rows")


PINS = [pin_golden, pin_score_library, pin_topk_bruteforce,
        pin_groups_bruteforce, pin_select_bruteforce, pin_renorm_identities, pin_scale_linearity,
        pin_backward_fd, pin_aux_backward_fd, pin_backward_invariants,
        pin_rows_independent, pin_margin, pin_tokens_per_expert,
        pin_aux_loss_closed_forms, pin_aux_loss_fd, pin_route_maps_bruteforce,
        pin_route_maps_vs_topk, pin_shared_gate_library, pin_shared_gate_invariants]
