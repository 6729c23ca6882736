"""Pins for the oracle's backward (gradients of L = sum <o_t, dO_t> + <S_T, dST>).

The recurrence of "Semidirect Fourier Delta Attention" §1 eq. (1) with the
read-out of §3 eq. (14) makes L a polynomial of degree at most two in any one
scalar input (S_t is linear in alpha_t, beta_t, v_t and in S_{t-1}, quadratic
in k_t through k k^T, and o_t is linear in q_t and S_t).  A central difference
is therefore exact for every scalar, up to rounding, once the perturbed inputs
are exactly representable: the inputs here lie on a 2^-12 grid and the step is
2^-6.  That checks every gradient entry against the forward oracle alone.  The
closed forms and Euler identities below check the same code from two more
directions (beta = 0 reduces the recurrence to a diagonal one, and L is
homogeneous of degree one in q and in (v, S0)).
"""
import numpy as np
import pytest

GRID = 2.0 ** -12
H_STEP = 2.0 ** -6


def _grid(x):
    return np.round(np.asarray(x, dtype=np.float64) / GRID) * GRID


def _inputs(seed, B=1, T=6, H=2, Dk=4, Dv=3, ckda=True, s0=True, dst=True):
    rng = np.random.default_rng(seed)
    q = _grid(rng.uniform(-1.5, 1.5, (B, T, H, Dk)))
    k = rng.standard_normal((B, T, H, Dk))
    k = _grid(k / np.linalg.norm(k, axis=-1, keepdims=True))
    v = _grid(rng.uniform(-1.5, 1.5, (B, T, H, Dv)))
    if ckda:
        alpha = _grid(rng.uniform(-1, 1, (B, T, H, Dk)))
        alpha[rng.random(alpha.shape) < 0.1] = -1.0
        alpha[rng.random(alpha.shape) < 0.1] = 0.0
        beta = _grid(rng.uniform(0, 2, (B, T, H)))
        beta[rng.random(beta.shape) < 0.15] = 2.0
        beta[rng.random(beta.shape) < 0.1] = 0.0
    else:
        alpha = _grid(rng.uniform(0.05, 1, (B, T, H, Dk)))
        beta = _grid(rng.uniform(0, 1, (B, T, H)))
    dO = _grid(rng.uniform(-1, 1, (B, T, H, Dv)))
    S0 = _grid(rng.uniform(-1, 1, (B, H, Dk, Dv))) if s0 else None
    dST = _grid(rng.uniform(-1, 1, (B, H, Dk, Dv))) if dst else None
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0), dO, dST


def _loss(oracle_lib, x, dO, dST):
    out, ST = oracle_lib.forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], nthreads=1)
    L = float(np.sum(out * dO))
    if dST is not None:
        L += float(np.sum(ST * dST))
    return L


GRAD = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta", "S0": "dS0"}


def _central(oracle_lib, x, dO, dST, name, idx):
    xp = {n: (None if a is None else a.copy()) for n, a in x.items()}
    xp[name][idx] += H_STEP
    lp = _loss(oracle_lib, xp, dO, dST)
    xp[name][idx] -= 2 * H_STEP
    lm = _loss(oracle_lib, xp, dO, dST)
    return (lp - lm) / (2 * H_STEP)


@pytest.mark.parametrize("seed,ckda", [(0, True), (1, True), (2, False)])
def test_backward_central_differences_every_entry(oracle_lib, seed, ckda):
    """Every gradient entry equals the (exact) central difference of L."""
    x, dO, dST = _inputs(seed, ckda=ckda)
    g = oracle_lib.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, x["S0"], dST,
                            nthreads=1)
    for name, gname in GRAD.items():
        a = x[name]
        for idx in np.ndindex(a.shape):
            fd = _central(oracle_lib, x, dO, dST, name, idx)
            assert abs(fd - g[gname][idx]) <= 1e-9 * (1.0 + abs(fd)), (name, idx, fd, g[gname][idx])


def test_backward_central_differences_across_checkpoints(oracle_lib):
    """T = 150 crosses the 64-token checkpoints of the state recomputation:
    sampled entries of every gradient against central differences."""
    x, dO, dST = _inputs(7, T=150, H=1, Dk=4, Dv=3)
    g = oracle_lib.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, x["S0"], dST,
                            nthreads=1)
    rng = np.random.default_rng(70)
    for name, gname in GRAD.items():
        a = x[name]
        flat = rng.choice(a.size, size=min(a.size, 12), replace=False)
        # always include the tokens on both sides of each checkpoint
        for idx in [np.unravel_index(f, a.shape) for f in flat]:
            fd = _central(oracle_lib, x, dO, dST, name, idx)
            assert abs(fd - g[gname][idx]) <= 1e-9 * (1.0 + abs(fd)), (name, idx)
    for t in (63, 64, 127, 128, 149):
        for name in ("alpha", "k", "beta"):
            idx = (0, t, 0) + ((1,) if name != "beta" else ())
            fd = _central(oracle_lib, x, dO, dST, name, idx)
            assert abs(fd - g[GRAD[name]][idx]) <= 1e-9 * (1.0 + abs(fd)), (name, idx)


@pytest.mark.parametrize("with_dst", [False, True])
def test_backward_euler_identities(oracle_lib, with_dst):
    """L is homogeneous of degree one in q (for dST = 0) and jointly in (v, S0):
    L = <dq, q> and L = <dv, v> + <dS0, S0>."""
    x, dO, dST = _inputs(11, T=9, H=2, Dk=5, Dv=4, dst=with_dst)
    g = oracle_lib.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, x["S0"], dST)
    L = _loss(oracle_lib, x, dO, dST)
    lin = float(np.sum(g["dv"] * x["v"]) + np.sum(g["dS0"] * x["S0"]))
    assert abs(L - lin) <= 1e-11 * (1 + abs(L))
    if not with_dst:
        assert abs(L - float(np.sum(g["dq"] * x["q"]))) <= 1e-11 * (1 + abs(L))


def test_backward_beta_zero_closed_form(oracle_lib):
    """beta = 0 leaves S_t = diag(Gamma_t) S0 with Gamma_t the running product of
    the gates (Prop. 2.1's diagonal recurrence at zero phase): then dk = dv = 0,
    dq_t = diag(Gamma_t) S0 dO_t, dS0 = sum_t diag(Gamma_t) q_t dO_t^T +
    diag(Gamma_T) dST, and dalpha_s = (product of the other gates) times the
    matching sums, written out with explicit products."""
    x, dO, dST = _inputs(5, T=7, H=1, Dk=4, Dv=3, ckda=False)
    x["beta"][:] = 0.0
    g = oracle_lib.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, x["S0"], dST)
    a = x["alpha"][0, :, 0, :]                      # [T, Dk]
    q = x["q"][0, :, 0, :]
    do = dO[0, :, 0, :]
    S0 = x["S0"][0, 0]
    sT = dST[0, 0]
    T, Dk = a.shape
    gam = np.cumprod(a, axis=0)                     # Gamma_t, inclusive
    assert np.abs(g["dk"]).max() == 0.0 and np.abs(g["dv"]).max() == 0.0
    np.testing.assert_allclose(g["dq"][0, :, 0, :], gam * (do @ S0.T), rtol=1e-13, atol=1e-14)
    dS0 = sum(np.outer(gam[t] * q[t], do[t]) for t in range(T)) + gam[-1][:, None] * sT
    np.testing.assert_allclose(g["dS0"][0, 0], dS0, rtol=1e-13, atol=1e-14)
    ref = np.zeros((T, Dk))
    for s in range(T):
        for c in range(Dk):
            acc = 0.0
            for t in range(s, T):
                others = np.prod([a[l, c] for l in range(t + 1) if l != s])
                acc += others * q[t, c] * (S0[c] @ do[t])
            acc += np.prod([a[l, c] for l in range(T) if l != s]) * (S0[c] @ sT[c])
            ref[s, c] = acc
    np.testing.assert_allclose(g["dalpha"][0, :, 0, :], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("chunk,T,ckda", [(16, 37, True), (8, 24, True), (16, 16, False), (4, 13, True)])
def test_chunked_backward_equals_sequential(oracle_lib, chunk, T, ckda):
    """The chunkwise gradient algebra (tests/chunk_model.py, the form the HIP
    backward computes) reproduces the oracle's token-by-token gradients: the
    chunked form changes cost, never the numbers ("Kimi Delta Attention: a
    bounded case study", Exercise 2)."""
    import chunk_model
    x, dO, dST = _inputs(21 + T, B=1, T=T, H=2, Dk=6, Dv=5, ckda=ckda)
    g = oracle_lib.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, x["S0"], dST)
    m = chunk_model.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, x["S0"], dST,
                             chunk=chunk)
    for name in g:
        scale = max(1.0, float(np.abs(g[name]).max()))
        np.testing.assert_allclose(m[name], g[name], rtol=0, atol=1e-9 * scale, err_msg=name)


# ---- backward through the input prologue ("Semidirect Fourier Delta
# Attention" §3, eqs. (15), (17), (18)) ------------------------------------------

PRO = dict(alpha_min=-1.0, alpha_max=1.0, beta_max=2.0, eps=0.0, normalize_q=True)


def _raw(seed, T=5, H=2, Dk=4, Dv=3):
    rng = np.random.default_rng(seed)
    g = lambda *s: _grid(rng.uniform(-1.5, 1.5, s))
    return dict(q=g(1, T, H, Dk), k=g(1, T, H, Dk), v=g(1, T, H, Dv), gate=g(1, T, H, Dk),
                beta=g(1, T, H), S0=g(1, H, Dk, Dv)), g(1, T, H, Dv), g(1, H, Dk, Dv)


def _loss_pro(oracle_lib, x, dO, dST, pro):
    out, ST = oracle_lib.forward_prologue(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["S0"],
                                          nthreads=1, **pro)
    return float(np.sum(out * dO) + np.sum(ST * dST))


@pytest.mark.parametrize("pro", [PRO, dict(alpha_min=0.05, alpha_max=0.95, beta_max=1.0,
                                                eps=0.125, normalize_q=False)])
def test_backward_prologue_matches_differences(oracle_lib, pro):
    """Every gradient of the raw inputs against a 4-point central difference
    (error O(h^4); the raw inputs lie on a 2^-12 grid, the step is 2^-7)."""
    x, dO, dST = _raw(3)
    g = oracle_lib.backward_prologue(x["q"], x["k"], x["v"], x["gate"], x["beta"], dO, x["S0"],
                                     dST, nthreads=1, **pro)
    names = {"q": "dq", "k": "dk", "v": "dv", "gate": "dgate", "beta": "dbeta_logit", "S0": "dS0"}
    h = 2.0 ** -7
    for name, gname in names.items():
        for idx in np.ndindex(x[name].shape):
            vals = []
            for m in (2, 1, -1, -2):
                xp = {n: a.copy() for n, a in x.items()}
                xp[name][idx] += m * h
                vals.append(_loss_pro(oracle_lib, xp, dO, dST, pro))
            fd = (-vals[0] + 8 * vals[1] - 8 * vals[2] + vals[3]) / (12 * h)
            assert abs(fd - g[gname][idx]) <= 2e-6 * (1 + abs(fd)), (name, idx, fd, g[gname][idx])


def test_backward_prologue_key_gradient_is_tangent(oracle_lib):
    """With eps = 0, k = k_raw / |k_raw| is invariant under scaling k_raw, so
    the gradient of k_raw is orthogonal to k_raw (likewise q_raw)."""
    x, dO, dST = _raw(8, T=7, Dk=6, Dv=5)
    g = oracle_lib.backward_prologue(x["q"], x["k"], x["v"], x["gate"], x["beta"], dO, x["S0"],
                                     dST, **PRO)
    for raw, gr in (("k", "dk"), ("q", "dq")):
        dots = np.sum(g[gr] * x[raw], axis=-1)
        scale = np.abs(g[gr]).max() * np.abs(x[raw]).max()
        assert np.abs(dots).max() <= 1e-12 * scale * x[raw].shape[-1]


# ---- backward of the phase variant ("Semidirect Fourier Delta Attention" §3
# eq. (13): the decay of channel pair p is alpha_p R(theta_p)) -------------------

def _phase(seed, T=6, H=2, Dk=4, Dv=3):
    rng = np.random.default_rng(seed)
    P = Dk // 2
    q = _grid(rng.uniform(-1.5, 1.5, (1, T, H, Dk)))
    k = rng.standard_normal((1, T, H, Dk))
    k = _grid(k / np.linalg.norm(k, axis=-1, keepdims=True))
    x = dict(q=q, k=k, v=_grid(rng.uniform(-1.5, 1.5, (1, T, H, Dv))),
             alpha=_grid(rng.uniform(-1, 1, (1, T, H, P))),
             theta=_grid(rng.uniform(-np.pi, np.pi, (1, T, H, P))),
             beta=_grid(rng.uniform(0, 2, (1, T, H))), S0=_grid(rng.uniform(-1, 1, (1, H, Dk, Dv))))
    return x, _grid(rng.uniform(-1, 1, (1, T, H, Dv))), _grid(rng.uniform(-1, 1, (1, H, Dk, Dv)))


def _loss_phase(oracle_lib, x, dO, dST):
    out, ST = oracle_lib.forward_phase(x["q"], x["k"], x["v"], x["alpha"], x["theta"], x["beta"],
                                       x["S0"], nthreads=1)
    return float(np.sum(out * dO) + np.sum(ST * dST))


@pytest.mark.parametrize("seed", [31, 32])
def test_backward_phase_matches_differences(oracle_lib, seed):
    """Every gradient of the phase variant against central differences of its
    forward: exact two-point differences for q, k, v, alpha, beta, S0 (L is a
    polynomial of degree at most two in each of them, the inputs lie on a 2^-12
    grid), a 4-point difference (error O(h^4), h = 2^-7) for theta, which
    enters through cos and sin."""
    x, dO, dST = _phase(seed)
    g = oracle_lib.backward_phase(x["q"], x["k"], x["v"], x["alpha"], x["theta"], x["beta"], dO,
                                  x["S0"], dST, nthreads=1)
    names = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "theta": "dtheta",
             "beta": "dbeta", "S0": "dS0"}
    for name, gname in names.items():
        h, steps = (2.0 ** -7, (2, 1, -1, -2)) if name == "theta" else (H_STEP, (1, -1))
        for idx in np.ndindex(x[name].shape):
            vals = []
            for m in steps:
                xp = {n: a.copy() for n, a in x.items()}
                xp[name][idx] += m * h
                vals.append(_loss_phase(oracle_lib, xp, dO, dST))
            if name == "theta":
                fd = (-vals[0] + 8 * vals[1] - 8 * vals[2] + vals[3]) / (12 * h)
                tol = 2e-6 * (1 + abs(fd))
            else:
                fd = (vals[0] - vals[1]) / (2 * h)
                tol = 1e-9 * (1 + abs(fd))
            assert abs(fd - g[gname][idx]) <= tol, (name, idx, fd, g[gname][idx])


def test_backward_phase_zero_is_kda(oracle_lib):
    """theta = 0: the plain backward with each pair's decay on both of its
    channels; the pair's alpha gradient is the sum of the two channels'."""
    x, dO, dST = _phase(33, T=9, H=2, Dk=6, Dv=4)
    x["theta"][:] = 0.0
    g = oracle_lib.backward_phase(x["q"], x["k"], x["v"], x["alpha"], x["theta"], x["beta"], dO,
                                  x["S0"], dST)
    a2 = np.repeat(x["alpha"], 2, axis=-1)
    r = oracle_lib.backward(x["q"], x["k"], x["v"], a2, x["beta"], dO, x["S0"], dST)
    for n in ("dq", "dk", "dv", "dbeta", "dS0"):
        np.testing.assert_allclose(g[n], r[n], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dalpha"], r["dalpha"][..., 0::2] + r["dalpha"][..., 1::2],
                               rtol=1e-12, atol=1e-12)


def _rotate_pairs(x, phi):
    """Rotate every channel pair (2p, 2p+1) of x [..., Dk] by phi [..., Dk/2]."""
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = c * a - s * b
    y[..., 1::2] = s * a + c * b
    return y


def test_backward_phase_by_rotated_inputs(oracle_lib):
    """The phase variant is the plain recurrence on q, k rotated by minus the
    running phase phi_t = theta_1 + ... + theta_t, with each pair's decay on
    both channels, and its final state rotated by phi_T.  So the gradients
    follow from the plain backward on those inputs: dq_t, dk_t rotated back by
    phi_t, the alpha gradients of a pair summed, and dtheta_s the sum over
    t >= s of d L / d phi_t, where d L / d phi_t = <dq'_t, -J q'_t> +
    <dk'_t, -J k'_t> (+ <dS_T, J S_T> at the last token), J the rotation by a
    right angle."""
    x, dO, dST = _phase(34, T=11, H=2, Dk=6, Dv=4)
    g = oracle_lib.backward_phase(x["q"], x["k"], x["v"], x["alpha"], x["theta"], x["beta"], dO,
                                  x["S0"], dST)
    phi = np.cumsum(x["theta"].astype(np.float64), axis=1)
    qr, kr = _rotate_pairs(x["q"], -phi), _rotate_pairs(x["k"], -phi)
    a2 = np.repeat(x["alpha"], 2, axis=-1)
    # the plain oracle takes fp32 inputs: compare in double through the exact
    # identity at the level of the rounded rotated inputs
    qr32, kr32 = qr.astype(np.float32).astype(np.float64), kr.astype(np.float32).astype(np.float64)
    out, STr = oracle_lib.forward(qr32, kr32, x["v"], a2, x["beta"], x["S0"])
    out_p, ST_p = oracle_lib.forward_phase(x["q"], x["k"], x["v"], x["alpha"], x["theta"],
                                           x["beta"], x["S0"])
    np.testing.assert_allclose(out, out_p, rtol=0, atol=1e-5)
    phiT = phi[:, -1]                                   # [1, H, P]
    ST_rot = np.swapaxes(_rotate_pairs(np.swapaxes(STr, -1, -2), phiT[:, :, None, :]), -1, -2)
    np.testing.assert_allclose(ST_rot, ST_p, rtol=0, atol=1e-5)
    dSTr = np.swapaxes(_rotate_pairs(np.swapaxes(dST, -1, -2), -phiT[:, :, None, :]), -1, -2)
    r = oracle_lib.backward(qr32, kr32, x["v"], a2, x["beta"], dO, x["S0"], dSTr)
    tol = dict(rtol=0, atol=1e-4)
    np.testing.assert_allclose(_rotate_pairs(r["dq"], phi), g["dq"], **tol)
    np.testing.assert_allclose(_rotate_pairs(r["dk"], phi), g["dk"], **tol)
    for n in ("dv", "dbeta", "dS0"):
        np.testing.assert_allclose(r[n], g[n], **tol)
    np.testing.assert_allclose(r["dalpha"][..., 0::2] + r["dalpha"][..., 1::2], g["dalpha"], **tol)

    def perp(d, u):        # <d, -J u> per pair = d_0 u_1 - d_1 u_0
        return d[..., 0::2] * u[..., 1::2] - d[..., 1::2] * u[..., 0::2]

    gphi = perp(r["dq"], qr32) + perp(r["dk"], kr32)
    # <dS'_T, J S'_T> per pair, summed over the value columns
    gphi[:, -1] += np.sum(dSTr[:, :, 1::2, :] * STr[:, :, 0::2, :]
                          - dSTr[:, :, 0::2, :] * STr[:, :, 1::2, :], axis=-1)
    dtheta = np.flip(np.cumsum(np.flip(gphi, axis=1), axis=1), axis=1)
    np.testing.assert_allclose(dtheta, g["dtheta"], **tol)
