"""The oracle pinned against brute force, closed forms and invariants (CPU).

The pages print no worked example, output values or error bound, so every pin
here comes from the mathematics of the method: see ``tests/pins.py``.  The
mutation tests plant plausible mistakes in a copy of the oracle's C source,
compile that copy on the CPU, and check that the pins reject it -- evidence
that the pins can tell a right oracle from a wrong one.
"""
from __future__ import annotations

import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_passes_pin(pin):
    pin(oracle.scan)


def test_linear_attention_pin_rejects_strict_mask():
    # The convention check: the A = 0 closed form with a strictly lower mask
    # (the reading y_t = c_t^T h_{t-1}) must NOT match the oracle.
    pr = pins.problem(41, b=1, L=12, nh=2, p=3, n=5, h0=True)
    pr["A"] = np.zeros_like(pr["A"])
    y, _, _ = oracle.scan(**pr)
    y_strict = pins.linear_attention(pr["x"], pr["dt"], pr["B"], pr["C"], pr["D"], pr["h0"], k=-1)
    assert pins.rel_err(y, y_strict) > 1e-2


def test_chunked_reference_with_strict_mask_disagrees():
    pr = pins.problem(5, L=9)
    y, _, _ = oracle.scan(**pr)
    yc, _ = pins.chunked(**pr, T=4, strict_mask=True)
    assert pins.rel_err(y, yc) > 1e-2


# ---------------------------------------------------------------------------
# helpers of the oracle package
# ---------------------------------------------------------------------------


def test_chunk_cumsum_matches_loop_definition():
    rng = np.random.default_rng(3)
    b, L, nh, T = 2, 37, 3, 8
    dt = rng.uniform(0, 2, (b, L, nh))
    A = -rng.uniform(1, 5, nh)
    G = oracle.chunk_cumsum(dt, A, T)
    nc = -(-L // T)
    assert G.shape == (b, nh, nc * T)
    for bi in range(b):
        for h in range(nh):
            for c in range(nc):
                run = 0.0
                for i in range(T):
                    t = c * T + i
                    if t < L:
                        run += A[h] * dt[bi, t, h]
                    assert abs(G[bi, h, t] - run) <= 1e-12 * max(1.0, abs(run))


def test_chunk_states_match_bruteforce():
    pr = pins.problem(8, b=2, L=19, nh=4, p=3, n=5, g=2, h0=False)
    T = 6
    S = oracle.chunk_states(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], T)
    nc = -(-19 // T)
    assert S.shape == (2, 4, nc, 3, 5)
    for c in range(nc):
        sl = slice(c * T, min(19, (c + 1) * T))
        part = {k: (v[:, sl] if k in ("x", "dt", "B", "C") else v) for k, v in pr.items()}
        _, fr = pins.bruteforce(**part)
        assert pins.rel_err(S[:, :, c], fr) < 1e-11


def test_chunk_state_weights_reproduce_sequential_chunk_states():
    # summing every token's outer product x_t B_t^T with its weight must give
    # the state the sequential scan reaches from zero at the chunk end
    pr = pins.problem(10, b=2, L=23, nh=4, p=3, n=5, g=2, h0=False)
    T = 8
    Wt = oracle.chunk_state_weights(pr["dt"], pr["A"], T)
    nc = -(-23 // T)
    assert Wt.shape == (2, 4, nc * T)
    assert np.all(Wt[:, :, 23:] == 0.0)
    S = oracle.chunk_states(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], T)
    hpg = 4 // 2
    for c in range(nc):
        t1 = min(23, (c + 1) * T)
        for h in range(4):
            Bh = pr["B"][:, c * T:t1, h // hpg]                      # (b, t, n)
            xw = pr["x"][:, c * T:t1, h] * Wt[:, h, c * T:t1, None]   # (b, t, p)
            ref = np.einsum("btp,btn->bpn", xw, Bh)
            assert pins.rel_err(S[:, h, c], ref) < 1e-12
    # the chunk's last token enters with weight dt (no decay left)
    dtp = np.zeros((2, nc * T, 4))
    dtp[:, :23] = pr["dt"]
    for c in range(nc - 1):
        np.testing.assert_allclose(Wt[:, :, c * T + T - 1], dtp[:, c * T + T - 1], rtol=1e-15)


def test_chunk_start_states_match_chunked_reference():
    pr = pins.problem(9, b=1, L=21, nh=2, p=3, n=4, h0=True)
    T = 5
    ck = oracle.chunk_start_states(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], T, pr["h0"])
    assert ck.shape[2] == 5
    np.testing.assert_allclose(ck[:, :, 0], pr["h0"], rtol=0, atol=0)
    for c in range(1, 5):
        pre = {k: (v[:, : c * T] if k in ("x", "dt", "B", "C") else v) for k, v in pr.items()}
        _, fr = pins.chunked(**pre, T=T)
        assert pins.rel_err(ck[:, :, c], fr) < 1e-12


def test_oracle_rejects_bad_arguments():
    pr = pins.problem(1)
    with pytest.raises(ValueError):
        oracle.scan(pr["x"], pr["dt"], pr["A"][:1], pr["B"], pr["C"])
    with pytest.raises(ValueError):
        oracle.scan(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"][:, :, :, :2])


# ---------------------------------------------------------------------------
# golden fixtures
# ---------------------------------------------------------------------------

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_scalar_halving():
    """Hand-derived values (geometric series), see the fixture's citation."""
    with open(os.path.join(GOLDEN, "scalar_halving.json")) as f:
        g = json.load(f)
    L = len(g["y"])
    x = np.ones((1, L, 1, 1))
    dt = np.ones((1, L, 1))
    A = np.array([-np.log(2.0)])
    B = np.ones((1, L, 1, 1))
    C = np.ones((1, L, 1, 1))
    y, fin, _ = oracle.scan(x, dt, A, B, C)
    np.testing.assert_allclose(y[0, :, 0, 0], g["y"], rtol=1e-14)
    np.testing.assert_allclose(fin[0, 0, 0, 0], g["y"][-1], rtol=1e-14)


def test_golden_oracle_regression():
    """The oracle still produces what ``make_golden.py`` stored from it."""
    with open(os.path.join(GOLDEN, "oracle_tiny.json")) as f:
        g = json.load(f)
    inp = {k: (None if v is None else np.array(v, np.float64)) for k, v in g["inputs"].items()}
    y, fin, _ = oracle.scan(**inp)
    np.testing.assert_allclose(y, np.array(g["y"]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fin, np.array(g["final"]), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# mutation tests: planted mistakes must be caught by the pins
# ---------------------------------------------------------------------------

_SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

MUTANTS = {
    # readout with the pre-update state (the h_{t-1} reading)
    "readout_before_update": (
        "                    s[n] = decay * s[n] + (dt_t * B_t[n]) * x_tp;\n"
        "                    /* y_t = c_t^T h_t  (post-update state) */\n"
        "                    acc += C_t[n] * s[n];\n",
        "                    acc += C_t[n] * s[n];\n"
        "                    s[n] = decay * s[n] + (dt_t * B_t[n]) * x_tp;\n"),
    "dropped_skip": ("acc + d_skip * x_tp;", "acc;"),
    "decay_sign": ("exp(A[h] * dt_t)", "exp(-A[h] * dt_t)"),
    "group_mapping": ("const int64_t g = h / heads_per_group;",
                      "const int64_t g = h % ngroups;"),
    "transposed_initial_state": ("h0[((b * nheads + h) * headdim + p) * dstate + n]",
                                 "h0[((b * nheads + h) * dstate + n) * headdim + p]"),
    "missing_dt_in_input": ("(dt_t * B_t[n]) * x_tp", "B_t[n] * x_tp"),
    "decay_after_input": ("s[n] = decay * s[n] + (dt_t * B_t[n]) * x_tp;",
                          "s[n] = decay * (s[n] + (dt_t * B_t[n]) * x_tp);"),
    "checkpoint_off_by_one": ("t % ckpt_stride == 0", "(t + 1) % ckpt_stride == 0"),
    "y_uses_B_not_C": ("acc += C_t[n] * s[n];", "acc += B_t[n] * s[n];"),
}


# planted mistakes in the backward (adjoint) part of the oracle
BWD_MUTANTS = {
    "bwd_ddt_drops_decay_term": ("ddt[(b * seqlen + t) * nheads + h] = xLB + A[h] * alpha * inner;",
                                 "ddt[(b * seqlen + t) * nheads + h] = xLB;"),
    "bwd_carry_without_decay": ("lam[k] *= alpha;", "lam[k] *= 1.0;"),
    "bwd_dC_from_previous_state": ("sc += ht[p * N + n] * dyt[p];", "sc += hprev[p * N + n] * dyt[p];"),
    "bwd_dB_missing_dt": ("dBt[n] = dtv * sb;", "dBt[n] = sb;"),
    "bwd_dx_missing_skip": ("dxt[p] = dtv * lb + d_skip * dyt[p];", "dxt[p] = dtv * lb;"),
    "bwd_dA_missing_dt": ("dA_acc += dtv * alpha * inner;", "dA_acc += alpha * inner;"),
    "bwd_adjoint_uses_B_not_C": ("lam[p * N + n] += dyt[p] * Ct[n];", "lam[p * N + n] += dyt[p] * Bt[n];"),
    "bwd_group_sum_strided": ("for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {",
                              "for (int64_t h = g; h < nheads; h += ngroups) {"),
    "bwd_decay_inner_with_current_state": ("inner += lam[p * N + n] * hprev[p * N + n];",
                                           "inner += lam[p * N + n] * ht[p * N + n];"),
    "bwd_dD_uses_dx": ("dyx += dyt[p] * xt[p];", "dyx += dyt[p] * dxt[p];"),
}


def _compile_mutants(d, mutants):
    src = open(_SRC).read()
    libs = {}
    for name, (old, new) in mutants.items():
        assert old in src, "mutation target vanished: %s" % name
        cpath = d / (name + ".c")
        cpath.write_text(src.replace(old, new, 1))
        so = d / ("lib" + name + ".so")
        subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(cpath),
                        "-o", str(so), "-lm"], check=True)
        libs[name] = oracle.load_library(str(so))
    return libs


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    return _compile_mutants(tmp_path_factory.mktemp("mutants"), MUTANTS)


@pytest.fixture(scope="module")
def bwd_mutant_libs(tmp_path_factory):
    return _compile_mutants(tmp_path_factory.mktemp("bwd_mutants"), BWD_MUTANTS)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, mutant_libs):
    lib = mutant_libs[name]

    def scan(*a, **k):
        return oracle.scan_with(lib, *a, **k)

    failed = []
    for pin in pins.ALL_PINS:
        if pin is pins.pin_bruteforce_mp:
            continue  # slow; the fp64 brute force covers the same ground
        try:
            pin(scan)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught mutant %s" % name


def test_chunk_cb_brute_force_and_linear_attention():
    """chunk_cb against a double loop over token pairs, and -- with A = 0, the
    linear-attention special case of section "Mamba-2 architecture" -- the
    masked form sum_{j <= i} (C_i . B_j) dt_j x_j + D x_i of one chunk against
    the sequential recurrence."""
    rng = np.random.default_rng(11)
    b, L, nh, p, n, g, T = 2, 11, 2, 3, 5, 2, 8
    B = rng.standard_normal((b, L, g, n))
    C = rng.standard_normal((b, L, g, n))
    cb = oracle.chunk_cb(B, C, T)
    assert cb.shape == (b, 2, g, T, T)
    for bi in range(b):
        for c in range(2):
            for gi in range(g):
                for i in range(T):
                    for j in range(T):
                        ti, tj = c * T + i, c * T + j
                        want = 0.0
                        if ti < L and tj < L:
                            want = sum(C[bi, ti, gi, k] * B[bi, tj, gi, k] for k in range(n))
                        assert abs(cb[bi, c, gi, i, j] - want) < 1e-12
    # A = 0: one chunk of L tokens, no decay
    L1 = T
    x = rng.standard_normal((b, L1, nh, p))
    dt = rng.uniform(0.1, 1.0, (b, L1, nh))
    B1, C1 = B[:, :L1], C[:, :L1]
    D = rng.standard_normal(nh)
    y, _, _ = oracle.scan(x, dt, np.zeros(nh), B1, C1, D)
    cb1 = oracle.chunk_cb(B1, C1, T)[:, 0]
    hpg = nh // g
    for bi in range(b):
        for h in range(nh):
            W = np.tril(cb1[bi, h // hpg]) * dt[bi, :, h][None, :]
            want = W @ x[bi, :, h] + D[h] * x[bi, :, h]
            assert np.max(np.abs(y[bi, :, h] - want)) < 1e-10


def test_decode_step_single_token_closed_form():
    # One step from a state s: s' = exp(A dt) s + dt x B^T (per head row p),
    # y = s' C + D x -- written out with numpy einsum, from a random state.
    rng = np.random.default_rng(71)
    b, nh, p, n, g = 3, 4, 5, 6, 2
    x = rng.standard_normal((b, nh, p))
    dt = np.abs(rng.standard_normal((b, nh)))
    A = -np.abs(rng.standard_normal(nh))
    B = rng.standard_normal((b, g, n))
    C = rng.standard_normal((b, g, n))
    D = rng.standard_normal(nh)
    s = rng.standard_normal((b, nh, p, n))
    y, s1 = oracle.decode_step(x, dt, A, B, C, D, s)
    hg = np.arange(nh) // (nh // g)
    Bh, Ch = B[:, hg], C[:, hg]                       # (b, nh, n) per head
    decay = np.exp(A[None, :] * dt)[..., None, None]  # (b, nh, 1, 1)
    want_s = decay * s + (dt[..., None] * x)[..., None] * Bh[:, :, None, :]
    want_y = np.einsum("bhpn,bhn->bhp", want_s, Ch) + D[None, :, None] * x
    assert np.allclose(s1, want_s, rtol=1e-13, atol=1e-13)
    assert np.allclose(y, want_y, rtol=1e-12, atol=1e-12)


def test_decode_steps_chain_to_the_scan():
    # K single steps, each from the previous step's state, give the K-token
    # scan's outputs and final state (state continuity through one token).
    pr = pins.problem(73, b=2, L=9, nh=4, p=3, n=5, h0=True)
    y_ref, h_ref, _ = oracle.scan(**pr)
    s = pr["h0"]
    for t in range(pr["x"].shape[1]):
        y, s = oracle.decode_step(pr["x"][:, t], pr["dt"][:, t], pr["A"], pr["B"][:, t], pr["C"][:, t],
                                  pr["D"], s)
        assert np.allclose(y, y_ref[:, t], rtol=1e-12, atol=1e-12)
    assert np.allclose(s, h_ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# the backward pass
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("pin", pins.BWD_PINS, ids=lambda f: f.__name__)
def test_oracle_backward_passes_pin(pin):
    pin(oracle.scan_bwd, oracle.scan)


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_pins_catch_planted_mistake(name, bwd_mutant_libs):
    lib = bwd_mutant_libs[name]

    def scan_bwd(*a, **k):
        return oracle.scan_bwd_with(lib, *a, **k)

    failed = []
    for pin in pins.BWD_PINS:
        try:
            pin(scan_bwd, oracle.scan)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no backward pin caught mutant %s" % name


def test_backward_rejects_bad_arguments():
    pr, dy, dhT = pins.bwd_problem(271)
    with pytest.raises(ValueError):
        oracle.scan_bwd(**pr, dy=dy[:, :-1], dhT=dhT)
    with pytest.raises(ValueError):
        oracle.scan_bwd(**pr, dy=dy, dhT=dhT[:, :1])
