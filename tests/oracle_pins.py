"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, none of which re-types the oracle's own decay-then-correct loop.

Each pin is a plain function that raises AssertionError on failure and takes
an optional ``lib`` (an oracle library opened with oracle.open_library), so
that tests/test_oracle_pins.py can run every pin on the real oracle and
tests/test_oracle_mutants.py can run them on deliberately broken copies.

Pages cited (by title and section):
  [XT] xutianle.me, "Kimi Linear：用 KDA 重写长上下文注意力"
  [DS] docsaid.org, "Kimi Linear" (逐通道的遺忘)
"""
from __future__ import annotations

import json
import os

import numpy as np

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
f32 = np.float32


def _chain(q, k, v, g, beta, s0=None, *, l2=False, lib=None, ckpt_every=0, scale=1.0):
    """Run the oracle on one (sequence, head) chain given [T, d] arrays."""
    T, dk = q.shape
    dv = v.shape[1]
    o, fs, ck = O.kda_fwd(q.reshape(1, T, 1, dk).astype(f32), k.reshape(1, T, 1, dk).astype(f32),
                          v.reshape(1, T, 1, dv).astype(f32), g.reshape(1, T, 1, dk).astype(f32),
                          beta.reshape(1, T, 1).astype(f32),
                          None if s0 is None else s0.reshape(1, 1, dk, dv).astype(f32),
                          qk_l2norm=l2, ckpt_every=ckpt_every, scale=scale, nthreads=1,
                          lib=lib)
    ck = None if ck is None else ck[0, :, 0]
    return o[0, :, 0, :], fs[0, 0], ck


def _orthonormal(n, d, rng):
    """n rows that are orthonormal EXACTLY in fp32: rows of a Sylvester
    Hadamard matrix scaled by 1/sqrt(d) (d a power of 4, so the scale is a
    power of two), with random row choice, column permutation and signs."""
    assert d in (4, 16, 64) and n <= d
    H = np.array([[1.0]])
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    H = H / np.sqrt(d)
    rows = rng.permutation(d)[:n]
    cols = rng.permutation(d)
    signs = rng.choice([-1.0, 1.0], size=d)
    return (H[rows][:, cols] * signs[None, :]).copy()


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b)))
    assert err <= tol, f"{what}: relative error {err:.3e} > {tol:.1e}"


# --- P-a: the worked example of the forget-gate step ------------------------
def pin_worked_example(lib=None):
    """[DS §"KDA：把衰減拆到每個通道", two-channel table]: state (8, 6) becomes
    (4, 3) under scalar alpha 0.5 and (8, 0.6) under per-channel alpha
    (1.0, 0.1).  beta = 0 isolates the gate step."""
    with open(os.path.join(GOLDEN, "worked_example_decay.json")) as fh:
        ex = json.load(fh)
    s0 = np.array(ex["state_before"], dtype=f32).reshape(2, 1)
    q = np.array([[1.0, 0.0]], dtype=f32)
    k = np.array([[0.6, 0.8]], dtype=f32)
    v = np.array([[5.0]], dtype=f32)
    b = np.zeros((1,), dtype=f32)
    for alpha, want in ((ex["scalar_alpha"], ex["state_after_scalar"]),
                        (ex["channel_alpha"], ex["state_after_channel"])):
        a = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (2,))
        g = np.log(a).astype(f32).reshape(1, 2)
        o, fs, _ = _chain(q, k, v, g, b, s0, lib=lib)
        _close(fs[:, 0], want, 1e-6, f"worked example alpha={alpha}")
        _close(o[0], [want[0]], 1e-6, "worked example read-out")
    # The same table with d_v = 3: the gate must scale whole ROWS (key
    # channels) of the d_k x d_v state, never its columns.
    s3 = np.repeat(s0, 3, axis=1)
    g = np.log(np.asarray(ex["channel_alpha"])).astype(f32).reshape(1, 2)
    _, fs, _ = _chain(q, k, np.ones((1, 3), f32), g, b, s3, lib=lib)
    want = np.repeat(np.asarray(ex["state_after_channel"]).reshape(2, 1), 3, axis=1)
    _close(fs, want, 1e-6, "worked example, gate scales rows")


# --- P-b: scalar gate = Gated DeltaNet --------------------------------------
def pin_gdn(lib=None):
    """[XT §3]: with the same alpha in every channel KDA is Gated DeltaNet,
    S_t = alpha_t (I - beta_t k k^T) S_(t-1) + beta_t k v^T."""
    rng = np.random.default_rng(11)
    T, dk, dv = 12, 5, 3
    q = rng.standard_normal((T, dk)).astype(f32)
    k = rng.standard_normal((T, dk)).astype(f32)
    v = rng.standard_normal((T, dv)).astype(f32)
    a = rng.uniform(0.3, 1.0, T)
    g = np.repeat(np.log(a)[:, None], dk, axis=1).astype(f32)
    beta = rng.uniform(0.0, 1.0, T).astype(f32)
    s0 = rng.standard_normal((dk, dv)).astype(f32)
    o, fs, _ = _chain(q, k, v, g, beta, s0, lib=lib)
    S = s0.astype(np.float64)
    want = []
    for t in range(T):
        at = np.exp(np.float64(g[t, 0]))
        kt, bt = k[t].astype(np.float64), np.float64(beta[t])
        S = at * (S - bt * np.outer(kt, kt @ S)) + bt * np.outer(kt, v[t].astype(np.float64))
        want.append(S.T @ q[t].astype(np.float64))
    _close(o, np.array(want), 1e-12, "GDN outputs")
    _close(fs, S, 1e-12, "GDN final state")


# --- P-c: alpha = 1 is the delta rule ----------------------------------------
def pin_delta_rule(lib=None):
    """[XT §2]: with alpha = 1, S_t = (I - beta_t k_t k_t^T) S_(t-1) + beta_t k_t v_t^T."""
    rng = np.random.default_rng(12)
    T, dk, dv = 10, 4, 6
    q = rng.standard_normal((T, dk)).astype(f32)
    k = rng.standard_normal((T, dk)).astype(f32)
    v = rng.standard_normal((T, dv)).astype(f32)
    g = np.zeros((T, dk), f32)
    beta = rng.uniform(0.0, 1.0, T).astype(f32)
    s0 = rng.standard_normal((dk, dv)).astype(f32)
    o, fs, _ = _chain(q, k, v, g, beta, s0, lib=lib)
    S = s0.astype(np.float64)
    I = np.eye(dk)
    want = []
    for t in range(T):
        kt, bt = k[t].astype(np.float64), np.float64(beta[t])
        S = (I - bt * np.outer(kt, kt)) @ S + bt * np.outer(kt, v[t].astype(np.float64))
        want.append(q[t].astype(np.float64) @ S)
    _close(o, np.array(want), 1e-12, "delta rule outputs")
    _close(fs, S, 1e-12, "delta rule final state")


# --- P-d: orthonormal keys = (beta-weighted) linear attention ----------------
def pin_linear_attention(lib=None):
    """[XT §1]: linear attention reads o_t = sum_i v_i (k_i^T q_t).  With
    orthonormal keys, S_0 = 0 and alpha = 1 the delta rule's correction reads
    zero, so KDA gives o_t = sum_(i<=t) beta_i v_i (k_i^T q_t) exactly, and
    with beta = 1 plain linear attention."""
    rng = np.random.default_rng(13)
    T, dk, dv = 6, 16, 5
    k = _orthonormal(T, dk, rng).astype(f32)
    q = rng.standard_normal((T, dk)).astype(f32)
    v = rng.standard_normal((T, dv)).astype(f32)
    g = np.zeros((T, dk), f32)
    for beta in (np.ones(T, f32), rng.uniform(0.1, 1.0, T).astype(f32)):
        o, _, _ = _chain(q, k, v, g, beta, None, lib=lib)
        K, Q, V = (x.astype(np.float64) for x in (k, q, v))
        scores = np.tril(Q @ K.T) * beta.astype(np.float64)[None, :]
        _close(o, scores @ V, 1e-12, "linear attention outputs")
    # the read-out scale multiplies the output and nothing else
    o, fs1, _ = _chain(q, k, v, g, beta, None, lib=lib, scale=0.125)
    _close(o, 0.125 * (scores @ V), 1e-12, "scaled read-out")
    _, fs2, _ = _chain(q, k, v, g, beta, None, lib=lib)
    _close(fs1, fs2, 1e-15, "scale leaves the state alone")


def pin_l2_normalisation(lib=None):
    """[XT §6.2]: q and k are L2-normalised (unit norm) before the recurrence.
    Keys along orthonormal directions but of arbitrary length must then act
    as unit keys, and queries of any length as unit queries."""
    rng = np.random.default_rng(14)
    T, dk, dv = 5, 16, 3
    dirs = _orthonormal(T, dk, rng)
    lens = rng.uniform(1.0, 7.0, T)
    k = (dirs * lens[:, None]).astype(f32)
    q = rng.standard_normal((T, dk)).astype(f32) * 3.0
    v = rng.standard_normal((T, dv)).astype(f32)
    g = np.zeros((T, dk), f32)
    beta = rng.uniform(0.1, 1.0, T).astype(f32)
    o, _, _ = _chain(q, k, v, g, beta, None, l2=True, lib=lib)
    K = k.astype(np.float64) / np.linalg.norm(k.astype(np.float64), axis=1, keepdims=True)
    Q = q.astype(np.float64) / np.linalg.norm(q.astype(np.float64), axis=1, keepdims=True)
    scores = np.tril(Q @ K.T) * beta.astype(np.float64)[None, :]
    # the 1e-6 under the square root moves results by < 1e-6 relative here
    _close(o, scores @ v.astype(np.float64), 2e-6, "normalised linear attention")


# --- P-e: beta = 0 freezes the state; small beta -> linear attention ---------
def pin_frozen_and_small_beta(lib=None):
    rng = np.random.default_rng(15)
    T, dk, dv = 9, 6, 4
    q = rng.standard_normal((T, dk)).astype(f32)
    k = rng.standard_normal((T, dk)).astype(f32)
    v = rng.standard_normal((T, dv)).astype(f32)
    g = np.zeros((T, dk), f32)
    s0 = rng.standard_normal((dk, dv)).astype(f32)
    o, fs, _ = _chain(q, k, v, g, np.zeros(T, f32), s0, lib=lib)
    _close(fs, s0, 1e-15, "beta=0 keeps the state")
    _close(o, q.astype(np.float64) @ s0.astype(np.float64), 1e-13, "beta=0 read-out")
    # beta = eps, S_0 = 0: o / eps -> sum_(i<=t) v_i (k_i^T q_t) with error O(eps T)
    T = 40
    q = rng.standard_normal((T, dk)).astype(f32)
    k = rng.standard_normal((T, dk)).astype(f32)
    v = rng.standard_normal((T, dv)).astype(f32)
    eps = 1e-7
    o, _, _ = _chain(q, k, v, np.zeros((T, dk), f32), np.full(T, eps, f32), None, lib=lib)
    K, Q, V = (x.astype(np.float64) for x in (k, q, v))
    want = np.tril(Q @ K.T) @ V
    _close(o / np.float64(f32(eps)), want, 1e-4, "small-beta limit")


# --- P-f: exact retrieval -----------------------------------------------------
def pin_exact_retrieval(lib=None):
    """[XT §2]: with beta = 1 a delta-rule write makes the state read back
    exactly v_t at key k_t; with alpha = 1 and orthonormal keys later writes do
    not disturb earlier ones, whatever S_0 holds."""
    rng = np.random.default_rng(16)
    T, dk, dv = 12, 16, 5
    k = _orthonormal(T, dk, rng).astype(f32)
    q = rng.standard_normal((T, dk)).astype(f32)
    v = rng.standard_normal((T, dv)).astype(f32)
    s0 = rng.standard_normal((dk, dv)).astype(f32)
    _, fs, _ = _chain(q, k, v, np.zeros((T, dk), f32), np.ones(T, f32), s0, lib=lib)
    _close(k.astype(np.float64) @ fs, v, 1e-12, "exact retrieval S^T k_i = v_i")


# --- P-g: brute-force transition products -------------------------------------
def pin_transition_products(lib=None):
    """[XT §4]: A_t = (I - beta_t k_t k_t^T) Diag(alpha_t) and S_t = A_t S_(t-1)
    + beta_t k_t v_t^T; [XT §8]: unrolled, o_t sums over i of
    [q_t^T (A_t ... A_(i+1)) k_i] v_i -- with the write strength beta_i, which
    the page's unrolled formula leaves out -- plus the decayed initial state.
    Built from explicit d_k x d_k matrices with d_k != d_v."""
    rng = np.random.default_rng(17)
    T, dk, dv = 7, 5, 3
    q = rng.standard_normal((T, dk)).astype(f32)
    k = rng.standard_normal((T, dk)).astype(f32)
    v = rng.standard_normal((T, dv)).astype(f32)
    g = np.log(rng.uniform(0.3, 1.0, (T, dk))).astype(f32)
    beta = rng.uniform(0.0, 1.0, T).astype(f32)
    s0 = rng.standard_normal((dk, dv)).astype(f32)
    o, fs, _ = _chain(q, k, v, g, beta, s0, lib=lib)
    K, Q, V, S0 = (x.astype(np.float64) for x in (k, q, v, s0))
    B = beta.astype(np.float64)
    A = [(np.eye(dk) - B[t] * np.outer(K[t], K[t])) @ np.diag(np.exp(g[t].astype(np.float64)))
         for t in range(T)]

    def prod(i, t):  # A_t A_(t-1) ... A_(i+1), identity when i == t
        M = np.eye(dk)
        for j in range(i + 1, t + 1):
            M = A[j] @ M
        return M

    want_o = []
    for t in range(T):
        acc = (prod(-1, t) @ S0).T @ Q[t]
        for i in range(t + 1):
            acc = acc + (Q[t] @ prod(i, t) @ K[i]) * B[i] * V[i]
        want_o.append(acc)
    ST = prod(-1, T - 1) @ S0 + sum(prod(i, T - 1) @ np.outer(B[i] * K[i], V[i]) for i in range(T))
    _close(o, np.array(want_o), 1e-12, "unrolled read-out")
    _close(fs, ST, 1e-12, "product-form final state")


# --- P-h: the delta step is a gradient step ------------------------------------
def pin_gradient_step(lib=None):
    """[XT §2]: S_t = S~ - beta_t grad L(S~), L(S) = 1/2 ||S^T k_t - v_t||^2,
    taken at the gated state S~ = Diag(alpha_t) S_(t-1) [XT §3].  The gradient
    is taken by central differences (exact for a quadratic up to rounding)."""
    rng = np.random.default_rng(18)
    dk, dv = 5, 3
    q = rng.standard_normal((1, dk)).astype(f32)
    k = rng.standard_normal((1, dk)).astype(f32)
    v = rng.standard_normal((1, dv)).astype(f32)
    g = np.log(rng.uniform(0.3, 1.0, (1, dk))).astype(f32)
    beta = np.array([0.7], f32)
    s0 = rng.standard_normal((dk, dv)).astype(f32)
    _, fs, _ = _chain(q, k, v, g, beta, s0, lib=lib)
    St = np.exp(g[0].astype(np.float64))[:, None] * s0.astype(np.float64)
    kk, vv = k[0].astype(np.float64), v[0].astype(np.float64)

    def loss(S):
        r = S.T @ kk - vv
        return 0.5 * float(r @ r)

    h = 1e-3
    grad = np.zeros_like(St)
    for i in range(dk):
        for j in range(dv):
            E = np.zeros_like(St)
            E[i, j] = h
            grad[i, j] = (loss(St + E) - loss(St - E)) / (2 * h)
    _close(fs, St - np.float64(beta[0]) * grad, 1e-9, "gradient step")


# --- P-i: invariances -----------------------------------------------------------
def _rand_problem(rng, B, T, H, dk, dv, gate_shift=3.0):
    q = rng.standard_normal((B, T, H, dk)).astype(f32)
    k = rng.standard_normal((B, T, H, dk)).astype(f32)
    v = rng.standard_normal((B, T, H, dv)).astype(f32)
    z = rng.standard_normal((B, T, H, dk)) + gate_shift
    g = (-np.log1p(np.exp(-z))).astype(f32)  # logsigmoid
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(f32)
    return q, k, v, g, beta


def pin_invariances(lib=None):
    """Split-and-chain = whole; varlen = separate runs (with an empty
    sequence); head permutation equivariance; checkpoints = prefix runs;
    decode steps = prefill tokens; bf16 inputs widen exactly."""
    rng = np.random.default_rng(19)
    H, dk, dv = 3, 8, 6
    # varlen = separate dense runs, bitwise
    lens = [37, 0, 63, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, g, beta = _rand_problem(rng, 1, T, H, dk, dv)
    s0 = (0.5 * rng.standard_normal((len(lens), H, dk, dv))).astype(f32)
    o, fs, _ = O.kda_fwd(q, k, v, g, beta, s0, cu, nthreads=2, lib=lib)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        if L == 0:
            assert np.array_equal(fs[n], s0[n].astype(np.float64)), "empty sequence keeps state"
            continue
        o1, f1, _ = O.kda_fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b],
                              s0[n:n + 1], nthreads=1, lib=lib)
        assert np.array_equal(o[:, a:b], o1), f"varlen sequence {n} outputs"
        assert np.array_equal(fs[n], f1[0]), f"varlen sequence {n} state"
    # dense batch = varlen packing of equal lengths, bitwise
    qd, kd, vd, gd, bd = _rand_problem(rng, 2, 50, H, dk, dv)
    od, fd, _ = O.kda_fwd(qd, kd, vd, gd, bd, nthreads=2, lib=lib)
    cat = lambda x: x.reshape((1, -1) + x.shape[2:])
    ov, fv, _ = O.kda_fwd(cat(qd), cat(kd), cat(vd), cat(gd), cat(bd), None,
                          np.array([0, 50, 100], np.int32), nthreads=2, lib=lib)
    assert np.array_equal(od.reshape(ov.shape), ov) and np.array_equal(fd, fv), "batch = varlen"
    # head permutation equivariance, bitwise
    perm = np.array([2, 0, 1])
    op, fp, _ = O.kda_fwd(qd[:, :, perm], kd[:, :, perm], vd[:, :, perm], gd[:, :, perm],
                          bd[:, :, perm], nthreads=2, lib=lib)
    assert np.array_equal(op, od[:, :, perm]) and np.array_equal(fp, fd[:, perm]), "head perm"
    # checkpoints = prefix runs, bitwise
    T = 96
    q, k, v, g, beta = _rand_problem(rng, 1, T, H, dk, dv)
    _, fs, ck = O.kda_fwd(q, k, v, g, beta, ckpt_every=32, nthreads=2, lib=lib)
    assert ck.shape == (1, 3, H, dk, dv)
    for j in range(3):
        e = 32 * (j + 1)
        _, fj, _ = O.kda_fwd(q[:, :e], k[:, :e], v[:, :e], g[:, :e], beta[:, :e],
                             nthreads=1, lib=lib)
        assert np.array_equal(ck[0, j], fj[0]), f"checkpoint {j}"
    assert np.array_equal(ck[0, 2], fs[0]), "last checkpoint = final state"
    # split at a non-chunk boundary and chain through an fp32 state
    s0 = (0.1 * rng.standard_normal((1, H, dk, dv))).astype(f32)
    ow, fw, _ = O.kda_fwd(q, k, v, g, beta, s0, nthreads=2, lib=lib)
    c = 41
    o1, f1, _ = O.kda_fwd(q[:, :c], k[:, :c], v[:, :c], g[:, :c], beta[:, :c], s0,
                          nthreads=2, lib=lib)
    o2, f2, _ = O.kda_fwd(q[:, c:], k[:, c:], v[:, c:], g[:, c:], beta[:, c:],
                          f1.astype(f32), nthreads=2, lib=lib)
    _close(np.concatenate([o1, o2], axis=1), ow, 1e-6, "split outputs")
    _close(f2, fw, 1e-6, "split final state")
    # decode steps = prefill tokens, bitwise: [B, T, H, d] -> [T, B, H, d]
    tr = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1))
    od2, sd2 = O.kda_decode(tr(q), tr(k), tr(v), tr(g), tr(beta), s0, nthreads=2, lib=lib)
    assert np.array_equal(tr(od2), ow) and np.array_equal(sd2, fw), "decode = prefill"
    # bf16 inputs are widened exactly: same values as fp32 give the same bits
    import torch
    qb, kb, vb = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
    ob, fb, _ = O.kda_fwd(qb, kb, vb, g, beta, s0, nthreads=2, lib=lib)
    of, ff, _ = O.kda_fwd(qb.float(), kb.float(), vb.float(), g, beta, s0, nthreads=2, lib=lib)
    assert np.array_equal(ob, of) and np.array_equal(fb, ff), "bf16 widening"


# --- P-j: forgetting under the workloads' gate distribution --------------------
def pin_forgetting(lib=None, T=2048):
    """Under g = logsigmoid(N(0,1)+3) the influence of the initial state dies
    out: runs from different initial states agree to < 1e-12 relative after
    T = 2048 tokens (d = 128).  This licenses windowed spot checks of very long
    sequences that start from a zero state 2048 tokens before the window."""
    rng = np.random.default_rng(20)
    H, d = 2, 128
    q, k, v, g, beta = _rand_problem(rng, 1, T, H, d, d)
    _, fa, _ = O.kda_fwd(q, k, v, g, beta, None, nthreads=2, lib=lib)
    s1 = rng.standard_normal((1, H, d, d)).astype(f32)
    _, fb, _ = O.kda_fwd(q, k, v, g, beta, s1, nthreads=2, lib=lib)
    gap = np.max(np.abs(fa - fb)) / np.max(np.abs(fa))
    assert gap < 1e-12, f"forgetting gap {gap:.3e}"


# --- P-k: contractivity -----------------------------------------------------------
def pin_contractivity(lib=None):
    """With unit keys, beta in [0,1] and alpha in (0,1] every transition has
    spectral norm <= 1, so ||S_t||_F <= ||S_0||_F + sum_(i<=t) beta_i ||v_i||."""
    rng = np.random.default_rng(21)
    T, dk, dv = 64, 16, 8
    q, k, v, g, beta = (x[0, :, 0] for x in _rand_problem(rng, 1, T, 1, dk, dv, gate_shift=1.0))
    s0 = rng.standard_normal((dk, dv)).astype(f32)
    _, _, ck = _chain(q, k, v, g, beta, s0, l2=True, lib=lib, ckpt_every=1)
    bound = np.linalg.norm(s0.astype(np.float64)) + np.cumsum(
        beta.astype(np.float64) * np.linalg.norm(v.astype(np.float64), axis=1))
    norms = np.linalg.norm(ck.reshape(T, -1), axis=1)
    assert np.all(norms <= bound * (1 + 1e-12)), "contractivity bound violated"
    # and the state does change (a frozen oracle would pass the bound trivially)
    assert np.max(np.abs(ck[-1] - s0)) > 1e-3


# --- output epilogue: head-wise RMSNorm x sigmoid gate [XT §6.3] ----------------
def pin_gate_norm_worked_example(lib=None):
    """o = (3, 4): mean square 12.5; z = 0 gives the gate 1/2 exactly; w = (1, 2)."""
    o = np.array([[3.0, 4.0]], dtype=f32)
    z = np.zeros((1, 2), dtype=f32)
    w = np.array([1.0, 2.0], dtype=f32)
    y = O.gate_norm(o, z, w, eps=0.0, lib=lib)
    r = np.sqrt(12.5)
    _close(y, [[3.0 / r * 0.5, 4.0 / r * 2.0 * 0.5]], 1e-15, "gate-norm worked example")


def pin_gate_norm_unit_rms(lib=None):
    """With the gate saturated (z = 40: sigmoid = 1 - 4e-18), w = 1 and
    eps = 0, every row comes out with mean square exactly 1, whatever its
    scale; and the row's direction is kept."""
    rng = np.random.default_rng(21)
    o = (rng.standard_normal((6, 128)) * np.array([[1e-3], [1], [7], [1e3], [0.5], [2]])).astype(f32)
    z = np.full(o.shape, 40.0, dtype=f32)
    y = O.gate_norm(o, z, None, eps=0.0, lib=lib)
    ms = np.mean(y * y, axis=1)
    assert np.max(np.abs(ms - 1.0)) < 1e-13, f"rows not unit RMS: {ms}"
    cos = np.sum(y * o, axis=1) / np.sqrt(np.sum(y * y, axis=1) * np.sum(o.astype(np.float64) ** 2, axis=1))
    assert np.min(cos) > 1 - 1e-13, "normalisation changed a row's direction"


def pin_gate_norm_scale_invariance(lib=None):
    """RMSNorm ignores a positive scale of its row (eps = 0); the gate does not."""
    rng = np.random.default_rng(22)
    o = rng.standard_normal((8, 64)).astype(f32)
    z = rng.standard_normal((8, 64)).astype(f32)
    w = rng.uniform(0.5, 1.5, 64).astype(f32)
    y1 = O.gate_norm(o, z, w, eps=0.0, lib=lib)
    y2 = O.gate_norm((o * f32(8.0)).astype(f32), z, w, eps=0.0, lib=lib)  # exact power-of-2 scale
    _close(y2, y1, 1e-14, "scale invariance")


def pin_gate_norm_gate_symmetry(lib=None):
    """sigmoid(z) + sigmoid(-z) = 1: y(z) + y(-z) is the ungated normalised row,
    which the saturated gate (z = +40) also gives; sigmoid(0) = 1/2."""
    rng = np.random.default_rng(23)
    o = rng.standard_normal((5, 128)).astype(f32)
    z = (3 * rng.standard_normal((5, 128))).astype(f32)
    w = rng.uniform(0.5, 1.5, 128).astype(f32)
    y_pos = O.gate_norm(o, z, w, eps=1e-6, lib=lib)
    y_neg = O.gate_norm(o, -z, w, eps=1e-6, lib=lib)
    y_one = O.gate_norm(o, np.full(o.shape, 40.0, dtype=f32), w, eps=1e-6, lib=lib)
    y_half = O.gate_norm(o, np.zeros(o.shape, dtype=f32), w, eps=1e-6, lib=lib)
    _close(y_pos + y_neg, y_one, 1e-14, "gate symmetry")
    _close(2.0 * y_half, y_one, 1e-15, "sigmoid(0) = 1/2")


def pin_gate_norm_special_rows(lib=None):
    """A zero row stays zero with eps > 0; a constant row c gives
    c / sqrt(c^2 + eps) before weight and gate; bf16 inputs widen exactly."""
    o = np.zeros((3, 64), dtype=f32)
    o[1, :] = 0.25
    o[2, :] = -3.0
    z = np.full(o.shape, 40.0, dtype=f32)
    eps = 1e-2
    y = O.gate_norm(o, z, None, eps=eps, lib=lib)
    assert np.all(y[0] == 0.0), "zero row not zero"
    _close(y[1], np.full(64, 0.25 / np.sqrt(0.0625 + eps)), 1e-14, "constant row")
    _close(y[2], np.full(64, -3.0 / np.sqrt(9.0 + eps)), 1e-14, "negative constant row")
    import torch
    ob = torch.from_numpy(np.random.default_rng(24).standard_normal((4, 128)).astype(f32)).bfloat16()
    zb = torch.zeros(4, 128).bfloat16()
    yb = O.gate_norm(ob, zb, None, eps=1e-6, lib=lib)
    yf = O.gate_norm(ob.float(), zb.float(), None, eps=1e-6, lib=lib)
    assert np.array_equal(yb, yf), "bf16 inputs not widened exactly"


# --- ShortConv + Swish prologue [XT §6, §6.1; XD preprocessing list] ----------
def _silu(a):
    import torch
    return torch.nn.functional.silu(torch.from_numpy(np.asarray(a, np.float64))).numpy()


def pin_conv_shift(lib=None):
    """A filter with one tap at position W-1-s passes x_{t-s}: the output is
    swish of the input delayed by s tokens, zeros before the sequence."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((1, 12, 5)).astype(f32)
    for s_ in range(4):
        w = np.zeros((5, 4), dtype=f32)
        w[:, 3 - s_] = 1.0
        y, st = O.short_conv(x, w, lib=lib)
        ref = np.zeros_like(y)
        ref[:, s_:] = _silu(x[:, :12 - s_].astype(np.float64))
        _close(y, ref, 1e-15, f"shift by {s_}")
        _close(st, x[0, -3:].T, 0.0 + 1e-300, "carried state = last 3 inputs")


def pin_conv_numpy(lib=None):
    """Pre-activation = numpy's full convolution of each zero-padded channel
    with the reversed filter (a library routine), then SiLU; with bias."""
    rng = np.random.default_rng(32)
    B, T, C, W = 2, 37, 6, 4
    x = rng.standard_normal((B, T, C)).astype(f32)
    w = rng.standard_normal((C, W)).astype(f32)
    bias = rng.standard_normal(C).astype(f32)
    y, _ = O.short_conv(x, w, bias, lib=lib)
    pre = np.zeros((B, T, C))
    for b in range(B):
        for c in range(C):
            pre[b, :, c] = np.convolve(x[b, :, c].astype(np.float64),
                                       w[c, ::-1].astype(np.float64))[:T] + bias[c]
    _close(y, _silu(pre), 1e-14, "convolution + SiLU")


def pin_conv_continuation(lib=None):
    """Splitting a sequence and carrying the state reproduces the whole run;
    token-by-token steps (decode) do too; varlen packing (with an empty and a
    one-token sequence) equals separate runs with their own states."""
    rng = np.random.default_rng(33)
    T, C = 50, 8
    x = rng.standard_normal((1, T, C)).astype(f32)
    w = rng.standard_normal((C, 4)).astype(f32)
    s0 = rng.standard_normal((1, C, 3)).astype(f32)
    y, sf = O.short_conv(x, w, None, s0, lib=lib)
    y1, s1 = O.short_conv(x[:, :21], w, None, s0, lib=lib)
    y2, s2 = O.short_conv(x[:, 21:], w, None, s1.astype(f32), lib=lib)
    _close(np.concatenate([y1, y2], axis=1), y, 1e-15, "split and carry")
    _close(s2, sf, 1e-300, "carried state after split")
    st = s0
    ys = []
    for t in range(5):
        yt, st = O.short_conv(x[:, t:t + 1], w, None, st, lib=lib)
        st = st.astype(f32)
        ys.append(yt)
    _close(np.concatenate(ys, axis=1), y[:, :5], 1e-15, "token-by-token steps")
    lens = [7, 0, 1, 30]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    xs = rng.standard_normal((1, int(cu[-1]), C)).astype(f32)
    ss = rng.standard_normal((4, C, 3)).astype(f32)
    yv, sv = O.short_conv(xs, w, None, ss, cu, lib=lib)
    for n in range(4):
        a, b = cu[n], cu[n + 1]
        yn, sn = O.short_conv(xs[:, a:b], w, None, ss[n:n + 1], lib=lib)
        _close(yv[:, a:b], yn, 1e-300, f"varlen sequence {n}") if b > a else None
        _close(sv[n:n + 1], sn, 1e-300, f"varlen state {n}")


def pin_conv_bf16(lib=None):
    """bf16 inputs widen exactly."""
    import torch
    xb = torch.from_numpy(np.random.default_rng(34).standard_normal((1, 9, 16)).astype(f32)).bfloat16()
    w = np.random.default_rng(35).standard_normal((16, 4)).astype(f32)
    yb, _ = O.short_conv(xb, w, lib=lib)
    yf, _ = O.short_conv(xb.float(), w, lib=lib)
    assert np.array_equal(yb, yf), "bf16 not widened exactly"


# --- backward (gradient) pins ----------------------------------------------------
# [XT §5]: training runs the chunkwise form; the gradient of the operator is
# the vector-Jacobian product of its forward map.  These pins fix it from
# outside the reverse sweep: central differences of the (pinned) forward
# oracle, closed forms where the recurrence reduces to a read-out of a frozen
# state or to linear attention, and Euler's identity for the parts of the map
# that are homogeneous.

def _loss(q, k, v, g, beta, s0, do, dfin, cu=None, *, l2, scale, lib):
    o, fs, _ = O.kda_fwd(q, k, v, g, beta, s0, cu, qk_l2norm=l2, scale=scale, nthreads=1,
                         lib=lib)
    return float(np.sum(o * do) + np.sum(fs * dfin))


def _fd_check(inp, cu, *, l2, scale, lib, samples=None, seed=0, h=2.0 ** -12, tol=1e-6):
    """Central differences of the forward oracle against kda_bwd, every
    component of every input (or `samples` random ones per input)."""
    q, k, v, g, beta, s0, do, dfin = inp
    grads = O.kda_bwd(q, k, v, g, beta, do, s0, dfin, cu, qk_l2norm=l2, scale=scale,
                      nthreads=1, lib=lib)
    rng = np.random.default_rng(seed)
    args = [q, k, v, g, beta, s0]
    for ai, name in enumerate(("q", "k", "v", "g", "beta", "init_state")):
        x, grad = args[ai], grads[ai]
        if samples is None:
            idxs = list(np.ndindex(*x.shape))
        else:
            idxs = [tuple(int(rng.integers(0, n)) for n in x.shape) for _ in range(samples)]
        gmax = max(np.max(np.abs(grad)), 1e-30)
        for idx in idxs:
            plus, minus = list(args), list(args)
            xp, xm = x.copy(), x.copy()
            xp[idx] += f32(h)
            xm[idx] -= f32(h)
            plus[ai], minus[ai] = xp, xm
            fd = (_loss(*plus, do, dfin, cu, l2=l2, scale=scale, lib=lib) -
                  _loss(*minus, do, dfin, cu, l2=l2, scale=scale, lib=lib)) / (2 * h)
            err = abs(fd - grad[idx]) / gmax
            assert err <= tol, f"d{name}{idx}: fd {fd:.9e} vs {grad[idx]:.9e} ({err:.2e})"


def _bwd_problem(rng, B, T, H, dk, dv, N=None):
    q, k, v, g, beta = _rand_problem(rng, B, T, H, dk, dv)
    N = B if N is None else N
    s0 = (0.5 * rng.standard_normal((N, H, dk, dv))).astype(f32)
    do = rng.standard_normal((B, T, H, dv)).astype(f32)
    dfin = rng.standard_normal((N, H, dk, dv)).astype(f32)
    return q, k, v, g, beta, s0, do, dfin


def pin_bwd_finite_differences(lib=None):
    """Every input gradient equals the central difference of the forward map
    (error O(h^2) ~ 1e-8 at h = 2^-12): dense with the L2 norm and a read-out
    scale, varlen with an empty sequence and no norm, and one chain longer
    than the sweep's 64-token recompute block."""
    rng = np.random.default_rng(41)
    _fd_check(_bwd_problem(rng, 2, 5, 2, 4, 3), None, l2=True, scale=0.6, lib=lib)
    cu = np.array([0, 3, 3, 9], np.int32)
    _fd_check(_bwd_problem(rng, 1, 9, 1, 3, 2, N=3), cu, l2=False, scale=1.0, lib=lib)
    _fd_check(_bwd_problem(rng, 1, 70, 1, 3, 2), None, l2=True, scale=1.0, lib=lib,
              samples=25, seed=3)


def pin_bwd_frozen_state(lib=None):
    """beta = 0: nothing is written, S_t = Diag(prod_(s<=t) a_s) S_0 and
    o_t = scale S_t^T q_t.  With G_t = dL/dS_t = scale sum_(t'>=t) D(t,t') q_t' do_t'^T
    + D(t,T) dS_T (D the decay between the two tokens), the closed forms are
    dq_t = scale S_t do_t, dk = dv = 0, dg_t = rowsum(G_t o S_t),
    dbeta_t = (G_t^T k_t) . (v_t - S_t^T k_t) and dS_0 = Diag(a_0) G_0."""
    rng = np.random.default_rng(43)
    T, dk, dv, scale = 7, 5, 4, 0.8
    q, k, v, g, _ = (x[0, :, 0] for x in _rand_problem(rng, 1, T, 1, dk, dv, gate_shift=0.5))
    beta = np.zeros(T, f32)
    s0 = rng.standard_normal((dk, dv)).astype(f32)
    do = rng.standard_normal((T, dv)).astype(f32)
    dfin = rng.standard_normal((dk, dv)).astype(f32)
    r = O.kda_bwd(q.reshape(1, T, 1, dk), k.reshape(1, T, 1, dk), v.reshape(1, T, 1, dv),
                  g.reshape(1, T, 1, dk), beta.reshape(1, T, 1), do.reshape(1, T, 1, dv),
                  s0.reshape(1, 1, dk, dv), dfin.reshape(1, 1, dk, dv), qk_l2norm=False,
                  scale=scale, nthreads=1, lib=lib)
    dq, dkk, dvv, dg = (x[0, :, 0] for x in r[:4])
    db = r[4][0, :, 0]
    ds0 = r[5][0, 0]
    Q, K, V, Gl, S0, DO, DF = (x.astype(np.float64) for x in (q, k, v, g, s0, do, dfin))
    cum = np.cumsum(Gl, axis=0)                     # log decay from 0 through t
    S = [np.exp(cum[t])[:, None] * S0 for t in range(T)]
    Gt = []
    for t in range(T):
        acc = np.exp(cum[-1] - cum[t])[:, None] * DF
        for t2 in range(t, T):
            acc = acc + scale * np.exp(cum[t2] - cum[t])[:, None] * np.outer(Q[t2], DO[t2])
        Gt.append(acc)
    _close(dq, np.stack([scale * S[t] @ DO[t] for t in range(T)]), 1e-12, "frozen dq")
    assert np.max(np.abs(dkk)) == 0.0 and np.max(np.abs(dvv)) == 0.0, "frozen dk, dv"
    _close(dg, np.stack([np.sum(Gt[t] * S[t], axis=1) for t in range(T)]), 1e-12, "frozen dg")
    _close(db, np.array([(Gt[t].T @ K[t]) @ (V[t] - S[t].T @ K[t]) for t in range(T)]),
           1e-12, "frozen dbeta")
    _close(ds0, np.exp(cum[0])[:, None] * Gt[0], 1e-12, "frozen dS_0")


def pin_bwd_linear_attention(lib=None):
    """Orthonormal keys, alpha = 1, S_0 = 0, no norm: o_t = scale sum_(i<=t)
    beta_i v_i (k_i . q_t) (linear attention, [XT §1]), and every correction and
    its derivative in v, beta, q vanish, so dv_i = scale beta_i sum_(t>=i)
    (k_i . q_t) do_t + beta_i dS_T^T k_i, dq_t = scale sum_(i<=t) beta_i k_i (v_i . do_t),
    dbeta_i = scale sum_(t>=i) (k_i . q_t)(v_i . do_t) + k_i^T dS_T v_i."""
    rng = np.random.default_rng(47)
    T, dk, dv, scale = 6, 16, 5, 0.9
    k = _orthonormal(T, dk, rng).astype(f32)
    q = rng.standard_normal((T, dk)).astype(f32)
    v = rng.standard_normal((T, dv)).astype(f32)
    beta = rng.uniform(0.2, 1.0, T).astype(f32)
    g = np.zeros((T, dk), f32)
    do = rng.standard_normal((T, dv)).astype(f32)
    dfin = rng.standard_normal((dk, dv)).astype(f32)
    r = O.kda_bwd(q.reshape(1, T, 1, dk), k.reshape(1, T, 1, dk), v.reshape(1, T, 1, dv),
                  g.reshape(1, T, 1, dk), beta.reshape(1, T, 1), do.reshape(1, T, 1, dv),
                  None, dfin.reshape(1, 1, dk, dv), qk_l2norm=False, scale=scale, nthreads=1,
                  lib=lib)
    dq, dvv = r[0][0, :, 0], r[2][0, :, 0]
    db = r[4][0, :, 0]
    Q, K, V, Bt, DO, DF = (x.astype(np.float64) for x in (q, k, v, beta, do, dfin))
    M = np.triu(K @ Q.T)                               # M[i, t] = k_i . q_t for t >= i
    _close(dvv, scale * Bt[:, None] * (M @ DO) + Bt[:, None] * (K @ DF), 1e-12, "linear dv")
    _close(dq, scale * np.tril(DO @ V.T * Bt[None, :]) @ K, 1e-12, "linear dq")
    _close(db, scale * np.sum(M * (V @ DO.T), axis=1) + np.einsum("ic,cj,ij->i", K, DF, V),
           1e-12, "linear dbeta")


def pin_bwd_homogeneity(lib=None):
    """Euler's identity on homogeneous parts of the map: the recurrence is
    linear in (v, S_0) jointly, so sum v dv + sum S_0 dS_0 = L; without the
    norm o is linear in q, so sum q dq = sum do . o; with the norm o is
    unchanged by rescaling one token's q or k, so q_t . dq_t = k_t . dk_t = 0
    (up to the eps under the root)."""
    rng = np.random.default_rng(53)
    q, k, v, g, beta, s0, do, dfin = _bwd_problem(rng, 2, 40, 2, 8, 6)
    for l2 in (False, True):
        dq, dkk, dvv, _, _, ds0 = O.kda_bwd(q, k, v, g, beta, do, s0, dfin, qk_l2norm=l2,
                                            scale=0.7, lib=lib)
        o, fs, _ = O.kda_fwd(q, k, v, g, beta, s0, qk_l2norm=l2, scale=0.7, lib=lib)
        L = np.sum(o * do) + np.sum(fs * dfin)
        _close(np.sum(v * dvv) + np.sum(s0 * ds0), L, 1e-11, f"Euler in (v, S_0), l2={l2}")
        if not l2:
            _close(np.sum(q * dq), np.sum(o * do), 1e-11, "Euler in q")
        else:
            tq = np.sum(q.astype(np.float64) * dq, axis=-1)
            tk = np.sum(k.astype(np.float64) * dkk, axis=-1)
            ref = np.max(np.abs(q)) * np.max(np.abs(dq)) + np.max(np.abs(k)) * np.max(np.abs(dkk))
            assert np.max(np.abs(tq)) <= 1e-5 * ref and np.max(np.abs(tk)) <= 1e-5 * ref, \
                "scale invariance of the L2 norm"


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_frozen_state, pin_bwd_linear_attention,
            pin_bwd_homogeneity]

CONV_PINS = [pin_conv_shift, pin_conv_numpy, pin_conv_continuation, pin_conv_bf16]

GATE_NORM_PINS = [pin_gate_norm_worked_example, pin_gate_norm_unit_rms,
                  pin_gate_norm_scale_invariance, pin_gate_norm_gate_symmetry,
                  pin_gate_norm_special_rows]

ALL_PINS = [pin_worked_example, pin_gdn, pin_delta_rule, pin_linear_attention,
            pin_l2_normalisation, pin_frozen_and_small_beta, pin_exact_retrieval,
            pin_transition_products, pin_gradient_step, pin_invariances,
            pin_contractivity] + GATE_NORM_PINS + CONV_PINS + BWD_PINS
