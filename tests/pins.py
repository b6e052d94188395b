"""Independent references that pin the oracle to something other than itself.

Each reference is written from a different formulation than the oracle's
sequential loop, so that a plausible mistake in the oracle (a dropped term, a
wrong sign or index, a transposed operand, the wrong readout convention)
disagrees with at least one of them.  Page citations are to "Accelerating
Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA Tile",
section "Mamba-2 architecture", unless stated otherwise.

Every ``pin_*`` function takes a ``scan`` callable with the oracle's signature
``scan(x, dt, A, B, C, D=None, h0=None, ckpt_stride=0) -> (y, h_final, ckpt)``
and raises ``AssertionError`` when the callable disagrees with the pin.  The
tests apply them to the real oracle (must pass) and to mutants of it with a
planted mistake (must fail).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# small random problems
# ---------------------------------------------------------------------------


def problem(seed, b=1, L=9, nh=2, p=3, n=4, g=1, h0=True, a_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, L, nh, p))
    dt = np.log1p(np.exp(rng.standard_normal((b, L, nh))))      # > 0
    A = -np.exp(rng.uniform(0, np.log(4.0), nh)) * a_scale        # < 0
    B = rng.standard_normal((b, L, g, n))
    C = rng.standard_normal((b, L, g, n))
    D = rng.standard_normal(nh)
    H0 = rng.standard_normal((b, nh, p, n)) if h0 else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, h0=H0)


def _group(h, nh, g):
    return h // (nh // g)


def rel_err(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = max(np.sqrt(np.mean(ref ** 2)), 1e-300)
    return float(np.max(np.abs(a - ref)) / scale) if ref.size else 0.0


# ---------------------------------------------------------------------------
# P1: brute-force expansion of the decayed recurrence (the expansion of
# h_{t+T} into exponentially weighted outer products, generalised to every
# token and carrying an initial state), O(L^2) per (b, h).
# ---------------------------------------------------------------------------


def bruteforce(x, dt, A, B, C, D=None, h0=None):
    """y[t] = sum_{s<=t} exp(sum_{r=s+1..t} a_r) (c_t . dt_s B_s) x_s
              + exp(sum_{r<=t} a_r) c_t^T h0 + D x_t ;
    final = sum_s exp(sum_{r>s} a_r) dt_s x_s B_s^T + exp(sum_r a_r) h0."""
    b, L, nh, p = x.shape
    g, n = B.shape[2], B.shape[3]
    y = np.zeros((b, L, nh, p))
    fin = np.zeros((b, nh, p, n))
    for bi in range(b):
        for h in range(nh):
            gi = _group(h, nh, g)
            a = A[h] * dt[bi, :, h]
            for t in range(L):
                acc = np.zeros(p)
                for s in range(t + 1):
                    w = np.exp(a[s + 1: t + 1].sum())
                    acc += w * (C[bi, t, gi] @ (dt[bi, s, h] * B[bi, s, gi])) * x[bi, s, h]
                if h0 is not None:
                    acc += np.exp(a[: t + 1].sum()) * (h0[bi, h] @ C[bi, t, gi])
                if D is not None:
                    acc += D[h] * x[bi, t, h]
                y[bi, t, h] = acc
            st = np.zeros((p, n))
            for s in range(L):
                w = np.exp(a[s + 1:].sum())
                st += w * dt[bi, s, h] * np.outer(x[bi, s, h], B[bi, s, gi])
            if h0 is not None:
                st += np.exp(a.sum()) * h0[bi, h]
            fin[bi, h] = st
    return y, fin


def bruteforce_mp(x, dt, A, B, C, D=None, h0=None, dps=40):
    """The same expansion in pure-Python loops at ``dps`` decimal digits
    (mpmath), for tiny inputs; returns float64 arrays of the exact result."""
    import mpmath as mp
    mp.mp.dps = dps
    b, L, nh, p = x.shape
    g, n = B.shape[2], B.shape[3]
    M = lambda v: mp.mpf(float(v))  # noqa: E731  (inputs are exact binary64)
    y = np.zeros((b, L, nh, p))
    for bi in range(b):
        for h in range(nh):
            gi = _group(h, nh, g)
            a = [M(A[h]) * M(dt[bi, t, h]) for t in range(L)]
            for t in range(L):
                for pi in range(p):
                    acc = mp.mpf(0)
                    for s in range(t + 1):
                        w = mp.exp(mp.fsum(a[s + 1: t + 1]))
                        cb = mp.fsum(M(C[bi, t, gi, k]) * M(dt[bi, s, h]) * M(B[bi, s, gi, k])
                                     for k in range(n))
                        acc += w * cb * M(x[bi, s, h, pi])
                    if h0 is not None:
                        acc += mp.exp(mp.fsum(a[: t + 1])) * mp.fsum(
                            M(C[bi, t, gi, k]) * M(h0[bi, h, pi, k]) for k in range(n))
                    if D is not None:
                        acc += M(D[h]) * M(x[bi, t, h, pi])
                    y[bi, t, h, pi] = float(acc)
    return y


# ---------------------------------------------------------------------------
# P5: the chunked evaluation -- per chunk, the log-space state jump
#   h_next = exp(G_last) h + (exp(G_last - G) . B) X^T
# and the chunk output
#   Y = exp(G) C h + (exp(G - G^T) . (C B^T) . M) X + D X,
# M the causal mask that keeps the diagonal, G the inclusive cumsum of a_t
# inside the chunk, B the dt-scaled rows.  Plain fp64 numpy, any chunk size.
# ---------------------------------------------------------------------------


def chunked(x, dt, A, B, C, D=None, h0=None, T=4, strict_mask=False):
    b, L, nh, p = x.shape
    g, n = B.shape[2], B.shape[3]
    y = np.zeros((b, L, nh, p))
    fin = np.zeros((b, nh, p, n))
    for bi in range(b):
        for h in range(nh):
            gi = _group(h, nh, g)
            st = np.zeros((p, n)) if h0 is None else h0[bi, h].copy()
            for c0 in range(0, L, T):
                c1 = min(c0 + T, L)
                X = x[bi, c0:c1, h]                             # (t, p)
                Bc = dt[bi, c0:c1, h, None] * B[bi, c0:c1, gi]  # (t, n) dt-scaled rows
                Cc = C[bi, c0:c1, gi]                           # (t, n)
                G = np.cumsum(A[h] * dt[bi, c0:c1, h])          # inclusive
                k = -1 if strict_mask else 0
                mask = np.tril(np.ones((c1 - c0, c1 - c0), bool), k=k)
                diff = np.where(mask, G[:, None] - G[None, :], -np.inf)  # select before exp
                Lmat = np.exp(diff)
                Y = np.exp(G)[:, None] * (Cc @ st.T) + (Lmat * (Cc @ Bc.T)) @ X
                if D is not None:
                    Y = Y + D[h] * X
                y[bi, c0:c1, h] = Y
                st = np.exp(G[-1]) * st + ((np.exp(G[-1] - G)[:, None] * Bc).T @ X).T
            fin[bi, h] = st
    return y, fin


# ---------------------------------------------------------------------------
# P4: with A = 0 the model is causal linear attention:
#   Y = C h0^T + ((C (dt B)^T) . tril) X + D X   (tril keeps the diagonal)
# ---------------------------------------------------------------------------


def linear_attention(x, dt, B, C, D=None, h0=None, k=0):
    b, L, nh, p = x.shape
    g, n = B.shape[2], B.shape[3]
    y = np.zeros((b, L, nh, p))
    for bi in range(b):
        for h in range(nh):
            gi = _group(h, nh, g)
            Bs = dt[bi, :, h, None] * B[bi, :, gi]
            S = np.tril(C[bi, :, gi] @ Bs.T, k=k)
            Y = S @ x[bi, :, h]
            if h0 is not None:
                Y += C[bi, :, gi] @ h0[bi, h].T
            if D is not None:
                Y += D[h] * x[bi, :, h]
            y[bi, :, h] = Y
    return y


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------


def pin_bruteforce(scan, seeds=(1, 2, 3), tol=1e-11):
    for s in seeds:
        pr = problem(s, b=2, L=11, nh=4, p=3, n=5, g=2)
        y, fin, _ = scan(**pr)
        yr, fr = bruteforce(**pr)
        assert rel_err(y, yr) < tol, ("P1 y", rel_err(y, yr))
        assert rel_err(fin, fr) < tol, ("P1 final", rel_err(fin, fr))


def pin_bruteforce_mp(scan, tol=1e-13):
    pr = problem(11, b=1, L=6, nh=2, p=2, n=2, g=1)
    y, _, _ = scan(**pr)
    yr = bruteforce_mp(**pr)
    assert rel_err(y, yr) < tol, ("P1 mp", rel_err(y, yr))


def pin_d_only(scan):
    pr = problem(21, L=13, nh=3, p=4, n=5, h0=False)
    pr["B"] = np.zeros_like(pr["B"])
    y, fin, _ = scan(**pr)
    assert np.array_equal(y, pr["D"][None, None, :, None] * pr["x"]), "P2 B=0"
    assert np.array_equal(fin, np.zeros_like(fin)), "P2 B=0 final"
    pr = problem(22, L=13, nh=3, p=4, n=5, h0=True)
    pr["C"] = np.zeros_like(pr["C"])
    y, _, _ = scan(**pr)
    assert np.array_equal(y, pr["D"][None, None, :, None] * pr["x"]), "P2 C=0"


def pin_decayed_initial_state(scan, tol=1e-12):
    pr = problem(31, b=2, L=10, nh=3, p=3, n=5, h0=True)   # p != n catches transposes
    pr["x"] = np.zeros_like(pr["x"])
    y, fin, _ = scan(**pr)
    cs = np.cumsum(pr["A"][None, None, :] * pr["dt"], axis=1)   # (b, L, nh)
    yr = np.einsum("btn,bhpn->bthp", pr["C"][:, :, 0], pr["h0"]) * np.exp(cs)[..., None]
    fr = np.exp(cs[:, -1])[:, :, None, None] * pr["h0"]
    assert rel_err(y, yr) < tol, ("P3 y", rel_err(y, yr))
    assert rel_err(fin, fr) < tol, ("P3 final", rel_err(fin, fr))


def pin_linear_attention(scan, tol=1e-12):
    pr = problem(41, b=2, L=12, nh=4, p=3, n=5, g=2, h0=True)
    pr["A"] = np.zeros_like(pr["A"])
    y, _, _ = scan(**pr)
    yr = linear_attention(pr["x"], pr["dt"], pr["B"], pr["C"], pr["D"], pr["h0"])
    assert rel_err(y, yr) < tol, ("P4", rel_err(y, yr))


def pin_chunked(scan, tol=1e-12):
    for L in (1, 17, 37):
        pr = problem(50 + L, b=1, L=L, nh=2, p=3, n=4, g=1, h0=True)
        y, fin, _ = scan(**pr)
        for T in range(1, L + 1):
            yc, fc = chunked(**pr, T=T)
            assert rel_err(y, yc) < tol, ("P5 y", L, T, rel_err(y, yc))
            assert rel_err(fin, fc) < tol, ("P5 final", L, T, rel_err(fin, fc))


def pin_split_continuity(scan, tol=1e-12):
    pr = problem(61, b=2, L=15, nh=2, p=3, n=4, g=1, h0=True)
    y, fin, _ = scan(**pr)
    tok = ("x", "dt", "B", "C")
    for L1 in range(0, 16):
        first = {k: (v[:, :L1] if k in tok else v) for k, v in pr.items()}
        second = {k: (v[:, L1:] if k in tok else v) for k, v in pr.items()}
        y1, f1, _ = scan(**first)
        second["h0"] = f1
        y2, f2, _ = scan(**second)
        assert rel_err(np.concatenate([y1, y2], axis=1), y) < tol, ("P6 y", L1)
        assert rel_err(f2, fin) < tol, ("P6 final", L1)


def pin_group_expansion(scan):
    pr = problem(71, b=1, L=9, nh=6, p=2, n=3, g=3, h0=True)
    y, fin, _ = scan(**pr)
    rep = 6 // 3
    ex = dict(pr)
    ex["B"] = np.repeat(pr["B"], rep, axis=2)
    ex["C"] = np.repeat(pr["C"], rep, axis=2)
    y2, f2, _ = scan(**ex)
    assert np.array_equal(y, y2) and np.array_equal(fin, f2), "P7"


def pin_linearity(scan, tol=1e-12):
    pr = problem(81, b=1, L=10, nh=2, p=3, n=4, h0=True)
    y, _, _ = scan(**pr)
    q = problem(82, b=1, L=10, nh=2, p=3, n=4, h0=True)
    s = dict(pr, x=pr["x"] + q["x"], h0=pr["h0"] + q["h0"])
    y2, _, _ = scan(**dict(pr, x=q["x"], h0=q["h0"]))
    ys, _, _ = scan(**s)
    assert rel_err(ys, y + y2) < tol, "P8 additivity"
    ya, _, _ = scan(**dict(pr, x=3.5 * pr["x"], h0=3.5 * pr["h0"]))
    assert rel_err(ya, 3.5 * y) < tol, "P8 homogeneity"


def pin_scalar_geometric(scan, tol=1e-13):
    # N = P = 1, constant a and b_t x_t: h_t = alpha^(t+1) h0 + beta (1 - alpha^(t+1)) / (1 - alpha)
    L = 20
    alpha, dtv, Bv, xv, Cv, Dv, h0v = 0.5, 0.75, 1.3, -0.7, 2.0, 0.25, 3.0
    Av = np.log(alpha) / dtv
    x = np.full((1, L, 1, 1), xv)
    dt = np.full((1, L, 1), dtv)
    A = np.array([Av])
    B = np.full((1, L, 1, 1), Bv)
    C = np.full((1, L, 1, 1), Cv)
    D = np.array([Dv])
    h0 = np.full((1, 1, 1, 1), h0v)
    y, fin, _ = scan(x, dt, A, B, C, D, h0)
    t = np.arange(L)
    beta = dtv * Bv * xv
    h = alpha ** (t + 1) * h0v + beta * (1 - alpha ** (t + 1)) / (1 - alpha)
    assert rel_err(y[0, :, 0, 0], Cv * h + Dv * xv) < tol, "P9 y"
    assert rel_err(fin[0, 0, 0], [h[-1]]) < tol, "P9 final"


def pin_dt_zero(scan):
    pr = problem(91, b=1, L=8, nh=2, p=3, n=4, h0=True)
    pr["dt"] = np.zeros_like(pr["dt"])
    y, fin, _ = scan(**pr)
    yr = np.einsum("btn,bhpn->bthp", pr["C"][:, :, 0], pr["h0"]) + pr["D"][None, None, :, None] * pr["x"]
    assert rel_err(y, yr) < 1e-14, "P10 y"
    assert np.array_equal(fin, pr["h0"]), "P10 final"


def pin_checkpoints(scan, tol=1e-11):
    # The state before token k*stride equals the brute-force final state of the
    # prefix [0, k*stride).
    pr = problem(101, b=1, L=13, nh=2, p=3, n=4, g=1, h0=True)
    for stride in (1, 4, 5, 13, 20):
        _, _, ck = scan(**pr, ckpt_stride=stride)
        for k in range(ck.shape[2]):
            t = k * stride
            pre = {kk: (v[:, :t] if kk in ("x", "dt", "B", "C") else v) for kk, v in pr.items()}
            _, fr = bruteforce(**pre)
            assert rel_err(ck[:, :, k], fr) < tol, ("ckpt", stride, k)


ALL_PINS = [pin_bruteforce, pin_bruteforce_mp, pin_d_only, pin_decayed_initial_state,
            pin_linear_attention, pin_chunked, pin_split_continuity, pin_group_expansion,
            pin_linearity, pin_scalar_geometric, pin_dt_zero, pin_checkpoints]


# ---------------------------------------------------------------------------
# Pins of the backward pass (the gradients of <dy, y> + <dhT, h_final>).
#
# Every ``bpin_*`` takes ``scan_bwd`` with the signature of ``oracle.scan_bwd``
# and ``scan`` with the forward oracle's signature (the pinned forward above),
# and raises AssertionError on disagreement.  None of them restates the
# adjoint recurrence: they come from the forward map itself (its Jacobian
# columns, finite differences), from symmetries of the recurrence, and from
# the chain rule through the group and sequence structure.
# ---------------------------------------------------------------------------


def bwd_problem(seed, b=1, L=7, nh=2, p=3, n=4, g=1, h0=True):
    pr = problem(seed, b=b, L=L, nh=nh, p=p, n=n, g=g, h0=h0)
    rng = np.random.default_rng(seed + 1000)
    dy = rng.standard_normal(pr["x"].shape)
    dhT = rng.standard_normal((b, nh, p, n))
    return pr, dy, dhT


def _objective(scan, pr, dy, dhT):
    y, hT, _ = scan(**pr)
    return float(np.sum(y * dy) + np.sum(hT * dhT))


_GRAD_OF = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0"}


def bpin_affine_jacobians(scan_bwd, scan, tol=1e-11):
    # (y, h_final) is affine in each of x, B, C, D and h0 with the others
    # fixed, so each Jacobian column is f(theta + e_k) - f(theta) exactly (up
    # to rounding), and the gradient is the transposed Jacobian applied to
    # (dy, dhT).  Every element of every one of these gradients is checked.
    for seed, g, nh in ((201, 1, 2), (202, 2, 4)):
        pr, dy, dhT = bwd_problem(seed, b=2, L=5, nh=nh, p=2, n=3, g=g)
        gr = scan_bwd(**pr, dy=dy, dhT=dhT)
        base = _objective(scan, pr, dy, dhT)
        for name in ("x", "B", "C", "D", "h0"):
            v = pr[name]
            want = np.zeros(v.size)
            for k in range(v.size):
                e = np.zeros(v.size)
                e[k] = 1.0
                q = dict(pr)
                q[name] = v + e.reshape(v.shape)
                want[k] = _objective(scan, q, dy, dhT) - base
            got = gr[_GRAD_OF[name]].ravel()
            assert rel_err(got, want) < tol, ("affine jacobian", name, seed)


def bpin_finite_differences(scan_bwd, scan, tol=1e-7):
    # dt and A enter through exp(A dt): central differences with Richardson
    # extrapolation (error O(eps^4)) for every element of ddt and dA.
    pr, dy, dhT = bwd_problem(211, b=2, L=6, nh=3, p=2, n=3, g=1)
    gr = scan_bwd(**pr, dy=dy, dhT=dhT)
    for name in ("dt", "A"):
        v = pr[name]
        want = np.zeros(v.size)
        for k in range(v.size):
            e = np.zeros(v.size)
            e[k] = 1.0
            e = e.reshape(v.shape)

            def f(s):
                q = dict(pr)
                q[name] = v + s * e
                return _objective(scan, q, dy, dhT)

            h = 1e-3
            d1 = (f(h) - f(-h)) / (2 * h)
            d2 = (f(h / 2) - f(-h / 2)) / h
            want[k] = (4 * d2 - d1) / 3
        assert rel_err(gr[_GRAD_OF[name]].ravel(), want) < tol, ("finite differences", name)


def bpin_scaling_invariants(scan_bwd, scan, tol=1e-10):
    # Three one-parameter symmetries of the forward map give Euler identities
    # that tie different gradients together (d/ds of the objective at s = 1):
    #  1. (dt, A, B) -> (s dt, A / s, B / s) leaves A dt and dt B, hence every
    #     output, unchanged:    <dt, ddt> - <A, dA> - <B, dB> = 0 ;
    #  2. (x, B, D) -> (s x, B / s, D / s) leaves dt B x^T and D x unchanged:
    #                           <x, dx> - <B, dB> - <D, dD> = 0 ;
    #  3. (C, B, h0) -> (s C, B / s, h0 / s) scales every state by 1 / s and
    #     leaves y unchanged, so the objective changes by -<dhT, h_final>:
    #                           <C, dC> - <B, dB> - <h0, dh0> + <dhT, h_final> = 0 .
    for seed, g, nh in ((221, 1, 2), (222, 2, 4)):
        pr, dy, dhT = bwd_problem(seed, b=2, L=9, nh=nh, p=3, n=4, g=g)
        gr = scan_bwd(**pr, dy=dy, dhT=dhT)
        _, hT, _ = scan(**pr)

        def dot(a, b):
            return float(np.sum(np.asarray(a) * np.asarray(b)))

        scale = sum(abs(dot(pr[k], gr[_GRAD_OF[k]])) for k in _GRAD_OF) + 1.0
        i1 = dot(pr["dt"], gr["ddt"]) - dot(pr["A"], gr["dA"]) - dot(pr["B"], gr["dB"])
        i2 = dot(pr["x"], gr["dx"]) - dot(pr["B"], gr["dB"]) - dot(pr["D"], gr["dD"])
        i3 = dot(pr["C"], gr["dC"]) - dot(pr["B"], gr["dB"]) - dot(pr["h0"], gr["dh0"]) + dot(dhT, hT)
        for name, v in (("dt-A-B", i1), ("x-B-D", i2), ("C-B-h0", i3)):
            assert abs(v) / scale < tol, ("scaling invariant", name, v)


def bpin_single_token(scan_bwd, scan, tol=1e-12):
    # One token from a zero state: h = dt x B^T, y = dt (C . B) x + D x, so by
    # hand (per head; B and C of the head's group)
    #   dx  = dt (C . B) dy + D dy + dt dhT B      dD  = dy . x
    #   dC  = dt (dy . x) B                        dB  = dt (dy . x) C + dt dhT^T x
    #   ddt = (C . B)(dy . x) + x^T dhT B          dA  = 0
    # and, through h = exp(A dt) h0 + ... with h0 = 0,  dh0 = exp(A dt)(dhT + dy C^T).
    pr, dy, dhT = bwd_problem(231, b=2, L=1, nh=4, p=3, n=5, g=2, h0=False)
    gr = scan_bwd(**pr, dy=dy, dhT=dhT)
    x, dt, A, B, C, D = (pr[k] for k in ("x", "dt", "A", "B", "C", "D"))
    b, _, nh, p = x.shape
    g = B.shape[2]
    want = {k: np.zeros_like(gr[k]) for k in gr}
    for bi in range(b):
        for h in range(nh):
            gi = _group(h, nh, g)
            Bv, Cv, xv, dyv, d = B[bi, 0, gi], C[bi, 0, gi], x[bi, 0, h], dy[bi, 0, h], dt[bi, 0, h]
            cb, yx = float(Cv @ Bv), float(dyv @ xv)
            want["dx"][bi, 0, h] = d * cb * dyv + D[h] * dyv + d * (dhT[bi, h] @ Bv)
            want["dD"][h] += yx
            want["dC"][bi, 0, gi] += d * yx * Bv
            want["dB"][bi, 0, gi] += d * yx * Cv + d * (dhT[bi, h].T @ xv)
            want["ddt"][bi, 0, h] = cb * yx + float(xv @ dhT[bi, h] @ Bv)
            want["dh0"][bi, h] = np.exp(A[h] * d) * (dhT[bi, h] + np.outer(dyv, Cv))
    for k in want:
        assert rel_err(gr[k], want[k]) < tol or np.max(np.abs(gr[k] - want[k])) < 1e-14, ("single token", k)


def bpin_group_replication(scan_bwd, scan, tol=1e-12):
    # Sharing one B/C row among a group's heads is replication: with the rows
    # copied out to one group per head, the shared gradient is the sum of the
    # per-head copies' gradients (the chain rule through the copy), and every
    # other gradient is unchanged.
    pr, dy, dhT = bwd_problem(241, b=2, L=6, nh=4, p=2, n=3, g=2)
    gr = scan_bwd(**pr, dy=dy, dhT=dhT)
    hg = np.arange(4) // 2
    ex = dict(pr)
    ex["B"] = pr["B"][:, :, hg]
    ex["C"] = pr["C"][:, :, hg]
    ge = scan_bwd(**ex, dy=dy, dhT=dhT)
    for k in ("dB", "dC"):
        summed = np.stack([ge[k][:, :, hg == gi].sum(axis=2) for gi in range(2)], axis=2)
        assert rel_err(gr[k], summed) < tol, ("group replication", k)
    for k in ("dx", "ddt", "dA", "dD", "dh0"):
        assert rel_err(gr[k], ge[k]) < tol, ("group replication", k)


def bpin_split_continuity(scan_bwd, scan, tol=1e-12):
    # The sequence split at m: the second part starts from the first part's
    # final state, and the first part's backward receives the second part's
    # dh0 as its dhT.  Per-token gradients concatenate, dA and dD add, and the
    # whole sequence's dh0 is the first part's.
    pr, dy, dhT = bwd_problem(251, b=2, L=10, nh=2, p=3, n=4, g=1)
    gr = scan_bwd(**pr, dy=dy, dhT=dhT)
    m = 4
    tok = ("x", "dt", "B", "C")
    p1 = {k: (v[:, :m] if k in tok else v) for k, v in pr.items()}
    _, h_m, _ = scan(**p1)
    p2 = {k: (v[:, m:] if k in tok else v) for k, v in pr.items()}
    p2["h0"] = h_m
    g2 = scan_bwd(**p2, dy=dy[:, m:], dhT=dhT)
    g1 = scan_bwd(**p1, dy=dy[:, :m], dhT=g2["dh0"])
    for k in ("dx", "ddt", "dB", "dC"):
        assert rel_err(gr[k], np.concatenate([g1[k], g2[k]], axis=1)) < tol, ("split", k)
    for k in ("dA", "dD"):
        assert rel_err(gr[k], g1[k] + g2[k]) < tol, ("split", k)
    assert rel_err(gr["dh0"], g1["dh0"]) < tol, ("split", "dh0")


def bpin_empty_and_zero(scan_bwd, scan):
    # seqlen 0: the final state is h0, so dh0 = dhT and all else is zero.
    # dy = 0 and dhT = 0: every gradient is exactly zero.
    pr, dy, dhT = bwd_problem(261, b=1, L=0, nh=2, p=2, n=3)
    gr = scan_bwd(**pr, dy=dy, dhT=dhT)
    assert np.array_equal(gr["dh0"], dhT)
    for k in ("dA", "dD"):
        assert not np.any(gr[k])
    pr, dy, dhT = bwd_problem(262, b=1, L=5, nh=2, p=2, n=3)
    gr = scan_bwd(**pr, dy=np.zeros_like(dy), dhT=np.zeros_like(dhT))
    for k, v in gr.items():
        assert not np.any(v), ("zero cotangent", k)


BWD_PINS = [bpin_affine_jacobians, bpin_finite_differences, bpin_scaling_invariants, bpin_single_token,
            bpin_group_replication, bpin_split_continuity, bpin_empty_and_zero]
