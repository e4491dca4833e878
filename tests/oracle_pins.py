"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes an oracle library handle (``None`` = the real
oracle) and raises AssertionError if the oracle disagrees with the fact it
pins.  ``test_oracle_pins.py`` runs them on the oracle, and runs them again on
deliberately broken copies of the oracle source to show that each plausible
mistake fails at least one pin.

What pins what:
  scalar_golden      hand-worked dk = dv = 1 example (tests/golden/scalar_walk.json)
  matrix_form        S_t = a S (I - b k k^T) + b v k^T, o = S q with explicit
                     dv x dk matrices, dk != dv, unnormalised keys, several heads
  chunked_form       the WY/UT chunk algebra, written independently in numpy,
                     for chunk lengths 1, 3, 4, 16, 64 including a ragged tail
  pure_decay         beta = 0: h_T = exp(sum log_g) h0 and o_t = exp(G_t) h0^T q_t
  overwrite          alpha = beta = 1 with orthonormal keys: each value is written
                     exactly, retrieved exactly, and a rewrite keeps the last value
  state_carry        run(x1; h0) then run(x2; h1) equals run([x1; x2]; h0)
  linearity          (V, h0) -> (O, h_T) is linear for fixed q, k, gates
  contraction        ||h_t||_2 <= alpha_t ||h_{t-1}||_2 + beta_t ||v_t|| for unit keys
  packed             packed sequences (cu_seqlens) equal separate runs, bit for bit
  head_grouping      v-head vh reads k-head vh // (Hv / Hk)
  heads_subset       computing a subset of v-heads gives the same values
  empty              T = 0 leaves h0 unchanged
  decode             the K=4 verify/fold algebra (4x4 UT solve, fold of the first
                     na rows) in numpy equals the oracle's per-prefix states
  decode_rows        for K = 1, 2, 5, 8 rows, the oracle's outputs and per-prefix
                     states equal the token recurrence S <- a S (I - b k k^T) + b v k^T,
                     o = S q, applied row by row (the K = 1 step is its first row)

The gate/beta producer (the BA projection):
  ba_slots           where each output lands, against a table worked by hand from
                     the pages' index model (tests/golden/ba_slot_g3.json)
  ba_zero_input      x = 0: beta = 1/2 exactly, gate = -e^{a_log} ln(1 + e^{dt_bias})
  ba_special_values  softplus(0) = ln 2, softplus(z) -> z and e^{-|z|} for large |z|,
                     sigmoid(+-40) = 1 - e^{-40} and e^{-40}; e^{a_log} with a_log = ln 2
  ba_one_hot         a one-hot activation row picks one column of the weight
  ba_linearity       the pre-activations recovered from beta (logit) and from the
                     gate (inverse softplus) are linear in x and agree with each
                     other's group structure; extra row-stride columns are ignored
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(seed, B=2, T=11, Hk=2, Hv=4, dk=5, dv=3, unit=True, h0=True, gscale=0.3):
    rng = _rng(seed)
    mk = (lambda s: _unit(rng, s)) if unit else (lambda s: rng.standard_normal(s))
    q = mk((B, T, Hk, dk))
    k = mk((B, T, Hk, dk))
    v = rng.standard_normal((B, T, Hv, dv))
    log_g = -np.logaddexp(0.0, rng.standard_normal((B, T, Hv))) * gscale
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv))))
    h = rng.standard_normal((B, Hv, dk, dv)) * 0.5 if h0 else None
    return dict(q=q, k=k, v=v, log_g=log_g, beta=beta, h0=h)


def _close(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) / max(1.0, np.max(np.abs(b)))
    assert err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------

def pin_scalar_golden(lib=None):
    g = json.load(open(os.path.join(GOLDEN, "scalar_walk.json")))
    toks = g["tokens"]
    T = len(toks)
    sh = (1, T, 1, 1)
    q = np.array([t["q"] for t in toks]).reshape(sh)
    k = np.array([t["k"] for t in toks]).reshape(sh)
    v = np.array([t["v"] for t in toks]).reshape(sh)
    log_g = np.log(np.array([t["alpha"] for t in toks])).reshape(1, T, 1)
    beta = np.array([t["beta"] for t in toks]).reshape(1, T, 1)
    h0 = np.array([[[[g["h0"]]]]])
    out, hf = oracle.prefill(q, k, v, log_g, beta, h0, lib=lib)
    _close(out.ravel(), [t["o"] for t in toks], 1e-14, "scalar outputs")
    _close(hf.ravel(), [toks[-1]["S"]], 1e-14, "scalar final state")


def _matrix_form(c):
    """S is dv x dk; the state the oracle returns is h = S^T."""
    q, k, v, lg, be = c["q"], c["k"], c["v"], c["log_g"], c["beta"]
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    grp = Hv // Hk
    out = np.zeros((B, T, Hv, dv))
    hf = np.zeros((B, Hv, dk, dv))
    I = np.eye(dk)
    for b in range(B):
        for vh in range(Hv):
            kh = vh // grp
            S = c["h0"][b, vh].T.copy() if c["h0"] is not None else np.zeros((dv, dk))
            for t in range(T):
                kt = k[b, t, kh][:, None]
                a = np.exp(lg[b, t, vh])
                bt = be[b, t, vh]
                S = a * S @ (I - bt * kt @ kt.T) + bt * v[b, t, vh][:, None] @ kt.T
                out[b, t, vh] = S @ q[b, t, kh]
            hf[b, vh] = S.T
    return out, hf


def pin_matrix_form(lib=None):
    for seed, unit in ((1, False), (2, True)):
        c = _case(seed, B=2, T=9, Hk=2, Hv=4, dk=5, dv=3, unit=unit)
        out, hf = oracle.prefill(lib=lib, **c)
        ro, rh = _matrix_form(c)
        _close(out, ro, 1e-12, "matrix form outputs")
        _close(hf, rh, 1e-12, "matrix form state")


def _chunked_form(c, C):
    """WY/UT chunk algebra (own derivation, fp64), one (b, vh) at a time.

    Inside a chunk with start state h: G = cumsum(log_g), gamma = exp(G),
    Gamma_rs = exp(G_r - G_s) (s <= r), A = strict_lower(diag(beta) (Gamma o K K^T)),
    T = (I + A)^-1, U = T diag(beta) V, W = T diag(beta gamma) K, Delta = U - W h,
    O = diag(gamma) Q h + (lower_incl(Q K^T) o Gamma) Delta,
    h_next = gamma_L h + (diag(exp(G_L - G)) K)^T Delta.
    """
    q, k, v, lg, be = c["q"], c["k"], c["v"], c["log_g"], c["beta"]
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    grp = Hv // Hk
    out = np.zeros((B, T, Hv, dv))
    hf = np.zeros((B, Hv, dk, dv))
    for b in range(B):
        for vh in range(Hv):
            kh = vh // grp
            h = c["h0"][b, vh].copy() if c["h0"] is not None else np.zeros((dk, dv))
            for t0 in range(0, T, C):
                sl = slice(t0, min(T, t0 + C))
                K = k[b, sl, kh]
                Q = q[b, sl, kh]
                V = v[b, sl, vh]
                G = np.cumsum(lg[b, sl, vh])
                bt = be[b, sl, vh]
                gam = np.exp(G)
                L = K.shape[0]
                Gam = np.tril(np.exp(G[:, None] - G[None, :]))
                A = np.tril(bt[:, None] * Gam * (K @ K.T), -1)
                Tm = np.linalg.inv(np.eye(L) + A)
                U = Tm @ (bt[:, None] * V)
                W = Tm @ ((bt * gam)[:, None] * K)
                D = U - W @ h
                out[b, sl, vh] = gam[:, None] * (Q @ h) + (np.tril(Q @ K.T) * Gam) @ D
                h = gam[-1] * h + (np.exp(G[-1] - G)[:, None] * K).T @ D
            hf[b, vh] = h
    return out, hf


def pin_chunked_form(lib=None):
    c = _case(3, B=2, T=37, Hk=1, Hv=2, dk=8, dv=6)
    out, hf = oracle.prefill(lib=lib, **c)
    for C in (1, 3, 4, 16, 64):
        ro, rh = _chunked_form(c, C)
        _close(out, ro, 1e-12, f"chunked form C={C} outputs")
        _close(hf, rh, 1e-12, f"chunked form C={C} state")


def pin_pure_decay(lib=None):
    c = _case(4, B=1, T=13, Hk=1, Hv=2, dk=4, dv=3)
    c["beta"] = np.zeros_like(c["beta"])
    out, hf = oracle.prefill(lib=lib, **c)
    G = np.cumsum(c["log_g"][0], axis=0)  # [T, Hv]
    for vh in range(2):
        h0 = c["h0"][0, vh]
        _close(hf[0, vh], np.exp(G[-1, vh]) * h0, 1e-14, "decay state")
        exp_o = np.exp(G[:, vh])[:, None] * (c["q"][0, :, 0] @ h0)
        _close(out[0, :, vh], exp_o, 1e-14, "decay outputs")


def pin_overwrite(lib=None):
    rng = _rng(5)
    dk, dv, T = 6, 4, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T[:T]                                 # orthonormal rows
    v = rng.standard_normal((1, T, 1, dv))
    k = keys.reshape(1, T, 1, dk)
    q = k.copy()                                    # query each key as it is written
    h0 = rng.standard_normal((1, 1, dk, dv))
    ones = np.ones((1, T, 1))
    out, hf = oracle.prefill(q, k, v, np.zeros((1, T, 1)), ones, h0, lib=lib)
    _close(out[0, :, 0], v[0, :, 0], 1e-13, "retrieve as written")
    _close(keys @ hf[0, 0], v[0, :, 0], 1e-13, "retrieve after all writes")
    # write key 0 twice: the second value wins; other slots keep theirs
    k2 = np.concatenate([k, k[:, :1]], axis=1)
    v2 = np.concatenate([v, rng.standard_normal((1, 1, 1, dv))], axis=1)
    q2 = k2.copy()
    _, hf2 = oracle.prefill(q2, k2, v2, np.zeros((1, T + 1, 1)), np.ones((1, T + 1, 1)), h0, lib=lib)
    got = keys @ hf2[0, 0]
    _close(got[0], v2[0, -1, 0], 1e-13, "rewrite keeps the last value")
    _close(got[1:], v[0, 1:, 0], 1e-13, "rewrite leaves other keys")


def pin_state_carry(lib=None):
    c = _case(6, B=2, T=17, Hk=1, Hv=3, dk=5, dv=4)
    out, hf = oracle.prefill(lib=lib, **c)
    t1 = 7
    part = lambda sl: {kk: (vv[:, sl] if kk != "h0" else vv) for kk, vv in c.items()}
    c1 = part(slice(0, t1))
    o1, h1 = oracle.prefill(lib=lib, **c1)
    c2 = part(slice(t1, None))
    c2["h0"] = h1
    o2, h2 = oracle.prefill(lib=lib, **c2)
    _close(np.concatenate([o1, o2], axis=1), out, 1e-13, "carry outputs")
    _close(h2, hf, 1e-13, "carry state")


def pin_linearity(lib=None):
    c1 = _case(7, B=1, T=12, Hk=1, Hv=2, dk=4, dv=5)
    c2 = dict(c1)
    rng = _rng(8)
    c2["v"] = rng.standard_normal(c1["v"].shape)
    c2["h0"] = rng.standard_normal(c1["h0"].shape)
    a, b = 0.7, -1.3
    c3 = dict(c1)
    c3["v"] = a * c1["v"] + b * c2["v"]
    c3["h0"] = a * c1["h0"] + b * c2["h0"]
    o1, h1 = oracle.prefill(lib=lib, **c1)
    o2, h2 = oracle.prefill(lib=lib, **c2)
    o3, h3 = oracle.prefill(lib=lib, **c3)
    _close(o3, a * o1 + b * o2, 1e-12, "linear outputs")
    _close(h3, a * h1 + b * h2, 1e-12, "linear state")
    cz = dict(c1)
    cz["v"] = np.zeros_like(c1["v"])
    cz["h0"] = None
    oz, hz = oracle.prefill(lib=lib, **cz)
    assert np.all(oz == 0) and np.all(hz == 0), "no offset at zero input"


def pin_contraction(lib=None):
    c = _case(9, B=1, T=24, Hk=1, Hv=1, dk=6, dv=4, gscale=0.05)
    c["h0"] = c["h0"] * 10
    prev = np.linalg.norm(c["h0"][0, 0], 2)
    for t in range(c["q"].shape[1]):
        ct = {kk: (vv[:, : t + 1] if kk != "h0" else vv) for kk, vv in c.items()}
        _, h = oracle.prefill(lib=lib, **ct)
        cur = np.linalg.norm(h[0, 0], 2)
        bound = np.exp(c["log_g"][0, t, 0]) * prev + c["beta"][0, t, 0] * np.linalg.norm(c["v"][0, t, 0])
        assert cur <= bound * (1 + 1e-12), f"token {t}: {cur} > {bound}"
        prev = cur


def pin_packed(lib=None):
    rng = _rng(10)
    lens = [5, 0, 13, 1, 9]
    Hk, Hv, dk, dv = 2, 4, 4, 3
    seqs = [_case(20 + i, B=1, T=L, Hk=Hk, Hv=Hv, dk=dk, dv=dv) if L else None for i, L in enumerate(lens)]
    h0 = rng.standard_normal((len(lens), Hv, dk, dv))
    cat = lambda key: np.concatenate([s[key][0] for s in seqs if s is not None], axis=0)
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, hf = oracle.prefill(cat("q"), cat("k"), cat("v"), cat("log_g"), cat("beta"), h0,
                             cu_seqlens=cu, lib=lib)
    for i, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(hf[i], h0[i]), "empty sequence keeps its state"
            continue
        s = dict(seqs[i])
        s["h0"] = h0[i : i + 1]
        o, h = oracle.prefill(lib=lib, **s)
        assert np.array_equal(out[cu[i] : cu[i + 1]], o[0]), f"packed seq {i} outputs"
        assert np.array_equal(hf[i], h[0]), f"packed seq {i} state"


def pin_head_grouping(lib=None):
    c = _case(11, B=1, T=8, Hk=3, Hv=6, dk=4, dv=2)
    out, hf = oracle.prefill(lib=lib, **c)
    for vh in range(6):
        kh = vh // 2
        s = dict(q=c["q"][:, :, kh : kh + 1], k=c["k"][:, :, kh : kh + 1], v=c["v"][:, :, vh : vh + 1],
                 log_g=c["log_g"][:, :, vh : vh + 1], beta=c["beta"][:, :, vh : vh + 1],
                 h0=c["h0"][:, vh : vh + 1])
        ro, rh = _matrix_form(s)
        _close(out[:, :, vh : vh + 1], ro, 1e-12, f"v-head {vh} reads k-head {kh}")
        _close(hf[:, vh : vh + 1], rh, 1e-12, f"v-head {vh} state")


def pin_heads_subset(lib=None):
    c = _case(12, B=2, T=10, Hk=2, Hv=6, dk=4, dv=3)
    out, hf = oracle.prefill(lib=lib, **c)
    sub = [5, 0, 3]
    o2, h2 = oracle.prefill(heads=sub, lib=lib, **c)
    for vh in range(6):
        if vh in sub:
            assert np.array_equal(o2[:, :, vh], out[:, :, vh]) and np.array_equal(h2[:, vh], hf[:, vh])
        else:
            assert np.all(np.isnan(o2[:, :, vh])) and np.all(np.isnan(h2[:, vh]))


def pin_empty(lib=None):
    c = _case(13, B=2, T=0, Hk=1, Hv=2, dk=3, dv=3)
    out, hf = oracle.prefill(lib=lib, **c)
    assert out.size == 0
    assert np.array_equal(hf, c["h0"])
    c["h0"] = None
    _, hf = oracle.prefill(lib=lib, **c)
    assert np.all(hf == 0)


def _wy4(h0, q, k, v, lg, be):
    """Write-on-accept verify of K rows from state h0 (dk x dv), own algebra:
    A_rs = beta_r exp(G_r - G_s) k_r.k_s (s < r), Delta = (I + A)^-1 (diag(beta) V -
    diag(beta gamma) K h0), o_r = gamma_r h0^T q_r + sum_{s<=r} exp(G_r - G_s)(q_r.k_s) Delta_s,
    fold(na) = gamma_na h0 + sum_{s<na} exp(G_na - G_s) k_s Delta_s^T."""
    Kr = k.shape[0]
    G = np.cumsum(lg)
    gam = np.exp(G)
    Gam = np.tril(np.exp(G[:, None] - G[None, :]))
    A = np.tril(be[:, None] * Gam * (k @ k.T), -1)
    D = np.linalg.solve(np.eye(Kr) + A, be[:, None] * v - (be * gam)[:, None] * (k @ h0))
    o = gam[:, None] * (q @ h0) + (np.tril(q @ k.T) * Gam) @ D
    folds = [h0.copy()]
    for na in range(1, Kr + 1):
        folds.append(gam[na - 1] * h0 + (np.exp(G[na - 1] - G[:na])[:, None] * k[:na]).T @ D[:na])
    return o, folds


def pin_decode(lib=None):
    rng = _rng(14)
    B, K, Hk, Hv, dk, dv = 3, 4, 2, 4, 6, 5
    states = rng.standard_normal((B, Hv, dk, dv)) * 0.3
    q = _unit(rng, (B, K, Hk, dk))
    k = _unit(rng, (B, K, Hk, dk))
    v = rng.standard_normal((B, K, Hv, dv))
    gate = -np.logaddexp(0.0, rng.standard_normal((B, K, Hv))) * 0.3
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, K, Hv))))
    out, after = oracle.decode(states, q, k, v, gate, beta, lib=lib)
    for b in range(B):
        for vh in range(Hv):
            kh = vh // (Hv // Hk)
            o, folds = _wy4(states[b, vh], q[b, :, kh], k[b, :, kh], v[b, :, vh], gate[b, :, vh], beta[b, :, vh])
            _close(out[b, :, vh], o, 1e-12, "verify outputs")
            for na in range(K + 1):
                _close(after[b, na, vh], folds[na], 1e-12, f"fold na={na}")
            assert np.array_equal(after[b, 0, vh], states[b, vh]), "na = 0 is the untouched state"


def pin_decode_rows(lib=None):
    for K in (1, 2, 5, 8):
        rng = _rng(40 + K)
        B, Hk, Hv, dk, dv = 2, 1, 3, 7, 4
        states = rng.standard_normal((B, Hv, dk, dv)) * 0.3
        q = _unit(rng, (B, K, Hk, dk))
        k = _unit(rng, (B, K, Hk, dk))
        v = rng.standard_normal((B, K, Hv, dv))
        gate = -np.logaddexp(0.0, rng.standard_normal((B, K, Hv))) * 0.3
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, K, Hv))))
        out, after = oracle.decode(states, q, k, v, gate, beta, lib=lib)
        for b in range(B):
            for vh in range(Hv):
                S = states[b, vh].T.copy()   # S is dv x dk; the state h = S^T
                for r in range(K):
                    kt = k[b, r, 0][:, None]
                    S = np.exp(gate[b, r, vh]) * S @ (np.eye(dk) - beta[b, r, vh] * kt @ kt.T) \
                        + beta[b, r, vh] * v[b, r, vh][:, None] @ kt.T
                    _close(out[b, r, vh], S @ q[b, r, 0], 1e-12, f"K={K} row {r} output")
                    _close(after[b, r + 1, vh], S.T, 1e-12, f"K={K} state after {r + 1} rows")


# --------------------------------------------------------------------------
# The gate/beta producer.  Inputs are chosen so that each pre-activation
# y = x . w_n is known without the oracle (zero, one-hot, or a linear
# combination of runs), and the gating is checked at values whose results are
# closed forms.

def _ba(x, w, a_log, dt_bias, nv, G, lib):
    return oracle.ba_gates(x, w, a_log, dt_bias, nv, G, lib=lib)


def pin_ba_slots(lib=None):
    g = json.load(open(os.path.join(GOLDEN, "ba_slot_g3.json")))
    nv, G = g["nv"], g["vheads_per_group"]
    n, k = 2 * nv, 4
    y = 0.25 * np.arange(1, n + 1)          # distinct pre-activation per output
    w = np.zeros((n, k))
    w[:, 2] = y                              # x = e_2 selects column 2
    x = np.zeros((1, k))
    x[0, 2] = 1.0
    out = _ba(x, w, np.zeros(nv), np.zeros(nv), nv, G, lib)[0]
    for o, (kind, vh) in enumerate(g["slots"]):
        if kind == "beta":
            _close(out[nv + vh], 1.0 / (1.0 + np.exp(-y[o])), 1e-15, f"beta slot of output {o}")
        else:
            _close(out[vh], -np.logaddexp(0.0, y[o]), 1e-15, f"gate slot of output {o}")


def pin_ba_zero_input(lib=None):
    rng = _rng(71)
    nv, G, k = 8, 4, 32
    a_log = rng.standard_normal(nv)
    dt_bias = rng.standard_normal(nv) * 3.0
    out = _ba(np.zeros((3, k)), rng.standard_normal((2 * nv, k)), a_log, dt_bias, nv, G, lib)
    assert np.all(out[:, nv:] == 0.5), "beta of a zero pre-activation is exactly 1/2"
    gate = -np.exp(a_log) * np.log1p(np.exp(dt_bias))   # ln(1 + e^z) for moderate z
    for t in range(3):
        _close(out[t, :nv], gate, 1e-14, "gate of a zero input")
    assert np.all(out[:, :nv] < 0.0), "the log-decay is negative"


def pin_ba_special_values(lib=None):
    # one v-head per group, G = 1: output 2j is beta, 2j + 1 the gate of v-head j
    zs = np.array([0.0, 60.0, -60.0, 40.0])
    nv = zs.size
    w = np.zeros((2 * nv, 1))
    w[0::2, 0] = zs                          # beta pre-activations
    w[1::2, 0] = zs                          # gate pre-activations (dt_bias = 0)
    a_log = np.full(nv, np.log(2.0))         # e^{a_log} = 2
    out = _ba(np.ones((1, 1)), w, a_log, np.zeros(nv), nv, 1, lib)[0]
    gate, beta = out[:nv], out[nv:]
    _close(gate[0], -2.0 * np.log(2.0), 1e-15, "softplus(0) = ln 2")
    _close(gate[1], -2.0 * 60.0, 1e-15, "softplus(60) = 60 to fp64")
    assert abs(gate[2] - (-2.0 * np.exp(-60.0))) <= 1e-15 * 2.0 * np.exp(-60.0) * 10, "softplus(-60) = e^-60"
    assert beta[0] == 0.5
    assert abs(beta[3] - (1.0 - np.exp(-40.0))) <= 1e-16, "sigmoid(40) = 1 - e^-40"
    assert abs(beta[2] - np.exp(-60.0)) <= 1e-15 * np.exp(-60.0) * 10, "sigmoid(-60) = e^-60"


def pin_ba_one_hot(lib=None):
    rng = _rng(72)
    nv, G, k = 6, 2, 9
    w = rng.standard_normal((2 * nv, k))
    for j in (0, 4, k - 1):
        x = np.zeros((1, k))
        x[0, j] = 1.0
        out = _ba(x, w, np.zeros(nv), np.zeros(nv), nv, G, lib)[0]
        for o in range(2 * nv):
            grp, wi = divmod(o, 2 * G)
            if wi < G:
                _close(out[nv + grp * G + wi], 1.0 / (1.0 + np.exp(-w[o, j])), 1e-15, "one-hot beta")
            else:
                _close(out[grp * G + wi - G], -np.logaddexp(0.0, w[o, j]), 1e-15, "one-hot gate")


def _pre_activations(out, a_log, dt_bias, nv):
    """Invert the gating: y from beta (logit) and from the gate (inverse softplus)."""
    b = out[:, nv:]
    s = -out[:, :nv] / np.exp(a_log)                 # softplus(y + dt_bias) > 0
    with np.errstate(invalid="ignore", divide="ignore"):   # NaN where that fails: the pin then fails
        yb = np.log(b) - np.log1p(-b)
        yg = np.log(np.expm1(s)) - dt_bias
    return yg, yb


def pin_ba_linearity(lib=None):
    rng = _rng(73)
    nv, G, k, m = 6, 3, 40, 5
    w = rng.standard_normal((2 * nv, k)) * 0.2
    a_log = rng.standard_normal(nv) * 0.5
    dt_bias = rng.standard_normal(nv) * 0.5
    x1 = rng.standard_normal((m, k))
    x2 = rng.standard_normal((m, k))
    g1, b1 = _pre_activations(_ba(x1, w, a_log, dt_bias, nv, G, lib), a_log, dt_bias, nv)
    g2, b2 = _pre_activations(_ba(x2, w, a_log, dt_bias, nv, G, lib), a_log, dt_bias, nv)
    g3, b3 = _pre_activations(_ba(2.0 * x1 - x2, w, a_log, dt_bias, nv, G, lib), a_log, dt_bias, nv)
    _close(g3, 2.0 * g1 - g2, 1e-9, "gate pre-activation is linear in x")
    _close(b3, 2.0 * b1 - b2, 1e-9, "beta pre-activation is linear in x")
    # a wider row (row stride > k): the extra columns are not read
    wide = np.concatenate([x1, 1e6 * np.ones((m, 7))], axis=1)
    _close(_ba(wide, w, a_log, dt_bias, nv, G, lib), _ba(x1, w, a_log, dt_bias, nv, G, lib), 0.0,
           "columns beyond k")


ALL_PINS = [pin_scalar_golden, pin_matrix_form, pin_chunked_form, pin_pure_decay, pin_overwrite,
            pin_state_carry, pin_linearity, pin_contraction, pin_packed, pin_head_grouping,
            pin_heads_subset, pin_empty, pin_decode, pin_decode_rows, pin_ba_slots,
            pin_ba_zero_input, pin_ba_special_values, pin_ba_one_hot, pin_ba_linearity]
