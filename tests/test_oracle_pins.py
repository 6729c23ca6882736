"""Pins for the CPU oracle: what the pages and the mathematics fix.

Each test names the passage it follows.  Together they are chosen so that a
plausible slip in the oracle fails at least one of them:
  * decay dropped or applied after the write  -> channel-decay, overwrite pins
  * wrong sign / missing beta in the correction -> Householder, rotation, recall
  * read-out from the pre-update state          -> brute force, recall
  * transposed state or read-out               -> brute force with Dk != Dv
  * chunk-boundary or carried-state mistakes    -> chunked = sequential, linearity
"""
import json
import math
import os

import numpy as np
import pytest

import chunk_model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def run1(oracle_lib, S0, q, k, v, alpha, beta):
    """One (b, h) sequence: q,k,alpha [T,Dk]; v [T,Dv]; beta [T]; S0 [Dk,Dv]."""
    q, k, v, alpha = (np.asarray(x, dtype=np.float32)[None, :, None, :] for x in (q, k, v, alpha))
    beta = np.asarray(beta, dtype=np.float32)[None, :, None]
    S0 = None if S0 is None else np.asarray(S0, dtype=np.float32)[None, None]
    out, ST = oracle_lib.forward(q, k, v, alpha, beta, S0)
    return out[0, :, 0, :], ST[0, 0]


def rand_ckda(rng, T, Dk, Dv, unit_keys=True):
    q = rng.standard_normal((T, Dk))
    k = rng.standard_normal((T, Dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, Dv))
    alpha = rng.uniform(-1, 1, (T, Dk))
    beta = rng.uniform(0, 2, T)
    # values that must survive exactly: a few -1, 0 gates and beta = 2
    alpha[rng.random((T, Dk)) < 0.1] = -1.0
    alpha[rng.random((T, Dk)) < 0.1] = 0.0
    beta[rng.random(T) < 0.2] = 2.0
    f = lambda x: x.astype(np.float32).astype(np.float64)  # exact fp32 inputs
    return f(q), f(k), f(v), f(alpha), f(beta)


# --- Worked numbers: "Kimi Delta Attention: a bounded case study" ------------

def test_channel_decay_worked_example(oracle_lib):
    """Exercise 1 worked solution + §12.1: gate [0.9,0.2] keeps 0.9 and 0.2 of a
    unit trace; the [0.9,0.24] variant keeps 0.24 (+20%); row [10,10] -> [9,2]."""
    g = _golden("channel_decay.json")
    z = np.zeros((1, 2))
    # state S [Dk=2, Dv=1]; beta = 0 so only the gate acts; read channel 1 via q = e1
    out, S1 = run1(oracle_lib, np.array(g["initial_trace"])[:, None], np.array([[1.0, 0.0]]),
                   z, np.zeros((1, 1)), np.array([g["gate"]]), [0.0])
    assert np.allclose(S1[:, 0], g["after_one_step"], rtol=0, atol=1e-7)
    assert out[0, 0] == pytest.approx(g["after_one_step"][0], abs=1e-7)
    _, S1v = run1(oracle_lib, np.array(g["initial_trace"])[:, None], z, z, np.zeros((1, 1)),
                  np.array([g["variant_gate"]]), [0.0])
    assert np.allclose(S1v[:, 0], g["variant_after_one_step"], atol=1e-7)
    gain = 100.0 * (S1v[1, 0] / S1[1, 0] - 1.0)
    assert gain == pytest.approx(g["variant_gain_percent"], abs=1e-4)
    _, Sr = run1(oracle_lib, np.array(g["row"])[None, :].T, z, z, np.zeros((1, 1)),
                 np.array([g["gate"]]), [0.0])
    assert np.allclose(Sr[:, 0], g["row_after_decay"], atol=1e-5)


def test_half_life(oracle_lib):
    """Exercise 1 'First sort': half-life ln0.5/ln0.9 ~ 6.6 tokens vs ~0.43,
    a ~15x ratio.  Measured on the oracle's own trace of a unit state."""
    g = _golden("channel_decay.json")
    T = 8
    alpha = np.tile(np.array(g["gate"]), (T, 1))
    # read each channel separately through q = e1 / e2 on two copies of the run
    for ch, key in ((0, "half_life_tokens_channel1_approx"), (1, "half_life_tokens_channel2_approx")):
        q = np.zeros((T, 2)); q[:, ch] = 1.0
        out, _ = run1(oracle_lib, np.ones((2, 1)), q, np.zeros((T, 2)), np.zeros((T, 1)), alpha,
                      np.zeros(T))
        trace = out[:, 0]                     # trace[t-1] = gate^t
        per_step = trace[1] / trace[0]
        half_life = math.log(0.5) / math.log(per_step)
        assert round(half_life, 1 if ch == 0 else 2) == pytest.approx(g[key])
        if ch == 0:
            hl0 = half_life
            # crossing of 0.5 between the 6th and 7th token
            assert trace[5] > 0.5 > trace[6]
            assert trace[5] == pytest.approx(0.9 ** 6, rel=1e-6)
        else:
            hl1 = half_life
    assert round(hl0 / hl1) == g["half_life_ratio_approx"]


def test_delta_overwrite_then_fade(oracle_lib):
    """Exercise 2 reasoned solution: beta=1 correction on channel 2 gives exactly
    [4,4]; two steps of a 0.2 gate later it is 4*0.2^2 = 0.160.  The first gate
    is not 1 so that a write applied before the decay would be caught."""
    g = _golden("delta_overwrite.json")
    S0 = np.array([[3.0, -1.0], [7.0, 5.0]])
    k = np.zeros((3, 2)); k[0, g["key_channel"] - 1] = 1.0
    v = np.zeros((3, 2)); v[0] = g["value"]
    alpha = np.array([[0.5, 0.75], [1.0, g["fade_gate"]], [1.0, g["fade_gate"]]])
    beta = np.array([g["beta"], 0.0, 0.0])
    q = np.zeros((3, 2)); q[:, 1] = 1.0
    out, ST = run1(oracle_lib, S0, q, k, v, alpha, beta)
    assert np.array_equal(out[0], np.array(g["row_after_write"]))          # exact
    assert np.allclose(out[2], g["row_after_fade"], atol=1e-7)
    assert np.allclose(ST[0], S0[0] * 0.5)                                  # channel 1 only decays


def test_zero_gate_forgets(oracle_lib):
    """§12.1 quick check: a channel whose decay is zero forgets its previous
    content before the new update (exactly, for alpha = 0)."""
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((4, 3))
    alpha = np.array([[1.0, 0.0, 1.0, 1.0]])
    k = np.zeros((1, 4)); v = np.zeros((1, 3))
    _, S1 = run1(oracle_lib, S0, np.zeros((1, 4)), k, v, alpha, [0.0])
    assert np.all(S1[1] == 0.0)
    assert np.allclose(S1[[0, 2, 3]], S0[[0, 2, 3]].astype(np.float32))


# --- Closed forms: "Complex KDA" abstract --------------------------------------

def _transition(oracle_lib, k, alpha, beta):
    """The oracle's one-token transition matrix A_t, read off by running it on
    S0 = I with v = 0 (S_1 = A_t I)."""
    d = len(k)
    _, S1 = run1(oracle_lib, np.eye(d), np.zeros((1, d)), k[None], np.zeros((1, d)),
                 alpha[None], [beta])
    return S1


def test_householder(oracle_lib):
    """beta = 2 with a unit key and unit gates is the reflection I - 2kk^T:
    orthogonal, an involution, determinant -1."""
    rng = np.random.default_rng(7)
    k = rng.standard_normal(6); k /= np.linalg.norm(k)
    k = k.astype(np.float32).astype(np.float64)
    A = _transition(oracle_lib, k, np.ones(6), 2.0)
    n2 = float(k @ k)
    ref = np.eye(6) - 2.0 * np.outer(k, k)
    assert np.allclose(A, ref, atol=1e-12)
    assert np.allclose(A.T @ A, np.eye(6), atol=1e-6 * abs(1 - n2) + 1e-6)
    assert np.linalg.det(A) == pytest.approx(-1.0, abs=1e-6)
    assert np.allclose(A @ A, np.eye(6), atol=1e-6)


@pytest.mark.parametrize("d", [2, 5])
def test_rotation_from_two_reflections(oracle_lib, d):
    """One delta reflection (beta=2, k=(cos p, sin p, 0..)) after a gate
    reflection (alpha = (-1, 1, ..)) is the plane rotation R(2p) (+ identity);
    with p = pi/16, sixteen steps return the initial state."""
    p = math.pi / 16
    k = np.zeros(d); k[0], k[1] = math.cos(p), math.sin(p)
    alpha = np.ones(d); alpha[0] = -1.0
    kf = k.astype(np.float32).astype(np.float64)
    A = _transition(oracle_lib, kf, alpha, 2.0)
    ph = math.atan2(kf[1], kf[0])
    R = np.eye(d)
    R[:2, :2] = [[math.cos(2 * ph), -math.sin(2 * ph)], [math.sin(2 * ph), math.cos(2 * ph)]]
    nk = float(kf @ kf)
    assert np.allclose(A, R, atol=4 * abs(1 - nk) + 1e-12)
    T = 16
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((d, 3)).astype(np.float32)
    _, ST = run1(oracle_lib, S0, np.zeros((T, d)), np.tile(kf, (T, 1)), np.zeros((T, 3)),
                 np.tile(alpha, (T, 1)), np.full(T, 2.0))
    assert np.allclose(ST, S0, atol=1e-5)


def test_non_expansive(oracle_lib):
    """CKDA transitions with |alpha| <= 1, beta in [0,2] and unit keys are
    non-expansive: spectral norm <= 1 and the state norm never grows."""
    rng = np.random.default_rng(11)
    worst = 0.0
    for _ in range(300):
        d = 8
        k = rng.standard_normal(d); k /= np.linalg.norm(k)
        alpha = rng.uniform(-1, 1, d)
        beta = rng.uniform(0, 2)
        # exactly-normalised key in float64 so the bound is exact (inputs go in as
        # float32: renormalise the rounded key and accept its tiny norm defect)
        A = _transition(oracle_lib, k.astype(np.float32).astype(np.float64), alpha, beta)
        kf = k.astype(np.float32).astype(np.float64)
        slack = abs(1 - beta * (kf @ kf)) - 1 if beta * (kf @ kf) > 2 else 0.0
        worst = max(worst, np.linalg.norm(A, 2) - 1 - max(slack, 0))
    assert worst <= 1e-6
    q, k, _, alpha, beta = rand_ckda(rng, 64, 8, 4)
    S0 = rng.standard_normal((8, 4))
    norms = []
    S = S0.astype(np.float32)
    _, S = run1(oracle_lib, S, q[:1], k[:1], np.zeros((1, 4)), alpha[:1], beta[:1])
    prev = np.linalg.norm(S0.astype(np.float32))
    for t in range(64):
        _, S = run1(oracle_lib, S.astype(np.float32), q[t:t+1], k[t:t+1], np.zeros((1, 4)),
                    alpha[t:t+1], beta[t:t+1])
        n = np.linalg.norm(S)
        norms.append(n)
        assert n <= prev * (1 + 1e-5) + 1e-6
        prev = n


def test_orthogonal_case_preserves_norm(oracle_lib):
    """|alpha| = 1 with random signs and beta in {0, 2}, unit keys, v = 0: every
    transition is orthogonal, so ||S_t||_F stays at ||S_0||_F."""
    rng = np.random.default_rng(13)
    T, d = 200, 6
    k = rng.standard_normal((T, d)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    k = k.astype(np.float32).astype(np.float64)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    # only keys whose float32 rounding is (numerically) unit are meaningful here
    alpha = np.where(rng.random((T, d)) < 0.5, -1.0, 1.0)
    beta = np.where(rng.random(T) < 0.5, 0.0, 2.0)
    S0 = rng.standard_normal((d, 4)).astype(np.float32)
    q = np.zeros((T, d))
    out, ST = run1(oracle_lib, S0, q, k, np.zeros((T, 4)), alpha, beta)
    k32 = k.astype(np.float32).astype(np.float64)
    defect = np.max(np.abs(np.sum(k32 * k32, axis=1) - 1))
    assert np.linalg.norm(ST) == pytest.approx(np.linalg.norm(S0), rel=4 * T * defect + 1e-12)


# --- Prop. 2.1 of "Semidirect Fourier Delta Attention" --------------------------

def test_beta_zero_is_diagonal_recurrence(oracle_lib):
    """beta = 0 reduces the update to S_t = diag(alpha_t) S_{t-1} (Prop. 2.1,
    real case), so S_T = diag(prod alpha) S_0."""
    rng = np.random.default_rng(17)
    q, k, v, alpha, _ = rand_ckda(rng, 20, 7, 5)
    S0 = rng.standard_normal((7, 5)).astype(np.float32).astype(np.float64)
    out, ST = run1(oracle_lib, S0, q, k, v, alpha, np.zeros(20))
    prod = np.prod(alpha, axis=0)
    assert np.allclose(ST, prod[:, None] * S0, rtol=1e-12, atol=1e-300)
    cum = np.cumprod(alpha, axis=0)
    ref_out = np.einsum("tc,cj->tj", q * cum, S0)
    assert np.allclose(out, ref_out, rtol=1e-12, atol=1e-14)


# --- Brute force: affine composition, §2.2 eq. (9)-(10) -----------------------

@pytest.mark.parametrize("seed", range(6))
def test_brute_force_affine_products(oracle_lib, seed):
    """Each token is S -> A_t S + B_t with A_t = (I - beta k k^T) diag(alpha),
    B_t = beta k v^T; composing the dense maps (eq. (10)) gives the state, and
    o_t = S_t^T q_t.  T <= 8, Dk != Dv to catch transposes."""
    rng = np.random.default_rng(100 + seed)
    T, Dk, Dv = 1 + seed % 8, 5, 3
    q, k, v, alpha, beta = rand_ckda(rng, T, Dk, Dv, unit_keys=seed % 2 == 0)
    S0 = rng.standard_normal((Dk, Dv)).astype(np.float32).astype(np.float64)
    out, ST = run1(oracle_lib, S0, q, k, v, alpha, beta)
    Acc, Bcc = np.eye(Dk), np.zeros((Dk, Dv))            # composed map (A_{t:1}, B)
    for t in range(T):
        At = (np.eye(Dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(alpha[t])
        Bt = beta[t] * np.outer(k[t], v[t])
        Acc, Bcc = At @ Acc, At @ Bcc + Bt                # (A_t,B_t) o (Acc,Bcc)
        St = Acc @ S0 + Bcc
        assert np.allclose(out[t], St.T @ q[t], rtol=1e-12, atol=1e-12)
    assert np.allclose(ST, Acc @ S0 + Bcc, rtol=1e-12, atol=1e-12)


# --- Write summary / linearity in S0: contribution 4 of the SFDA page -----------

def test_linearity_in_initial_state(oracle_lib):
    """The chunk's affine write summary is what the recursion produces from a
    zero state, so F(S0; v) = F(0; v) + F(S0; v = 0) for outputs and state."""
    rng = np.random.default_rng(23)
    q, k, v, alpha, beta = rand_ckda(rng, 40, 6, 4)
    S0 = rng.standard_normal((6, 4)).astype(np.float32).astype(np.float64)
    o_full, s_full = run1(oracle_lib, S0, q, k, v, alpha, beta)
    o_zero, s_zero = run1(oracle_lib, None, q, k, v, alpha, beta)
    o_hom, s_hom = run1(oracle_lib, S0, q, k, np.zeros_like(v), alpha, beta)
    assert np.allclose(o_full, o_zero + o_hom, rtol=1e-12, atol=1e-12)
    assert np.allclose(s_full, s_zero + s_hom, rtol=1e-12, atol=1e-12)


# --- Chunked = sequential: Exercise 2 of the case-study page --------------------

@pytest.mark.parametrize("chunk,T", [(1, 9), (2, 11), (16, 37), (64, 129), (16, 16)])
def test_chunked_equals_sequential(oracle_lib, chunk, T):
    rng = np.random.default_rng(chunk * 1000 + T)
    B, H, Dk, Dv = 1, 2, 8, 5
    qs, ks, vs, als, bes = [], [], [], [], []
    for _ in range(H):
        q, k, v, a, b = rand_ckda(rng, T, Dk, Dv)
        qs.append(q); ks.append(k); vs.append(v); als.append(a); bes.append(b)
    st = lambda xs: np.stack(xs, axis=1)[None]
    q, k, v, alpha = st(qs), st(ks), st(vs), st(als)
    beta = np.stack(bes, axis=1)[None]
    S0 = rng.standard_normal((B, H, Dk, Dv)).astype(np.float32).astype(np.float64)
    o_ref, s_ref = oracle_lib.forward(q, k, v, alpha, beta, S0)
    o_chk, s_chk = chunk_model.forward(q, k, v, alpha, beta, S0, chunk=chunk)
    scale = max(1.0, np.abs(o_ref).max())
    assert np.abs(o_chk - o_ref).max() <= 1e-12 * scale
    assert np.abs(s_chk - s_ref).max() <= 1e-12 * max(1.0, np.abs(s_ref).max())


# --- Library special case and associative recall ------------------------------

def test_identity_gates_no_write_is_a_plain_matmul(oracle_lib):
    """alpha = 1, beta = 0: the state never changes, so o_t = S0^T q_t, which is
    one library matrix product."""
    rng = np.random.default_rng(29)
    q = rng.standard_normal((30, 9)).astype(np.float32).astype(np.float64)
    S0 = rng.standard_normal((9, 4)).astype(np.float32).astype(np.float64)
    out, _ = run1(oracle_lib, S0, q, rng.standard_normal((30, 9)), rng.standard_normal((30, 4)),
                  np.ones((30, 9)), np.zeros(30))
    assert np.allclose(out, np.matmul(q, S0), rtol=1e-13, atol=1e-13)


def test_associative_recall(oracle_lib):
    """alpha = 1, beta = 1, orthonormal keys, zero state: each write stores v_j
    under k_j exactly (read-compare-correct), so querying k_j returns v_j."""
    d, dv = 8, 3
    keys = np.eye(d)[np.random.default_rng(31).permutation(d)]     # exactly orthonormal
    vals = np.random.default_rng(37).standard_normal((d, dv)).astype(np.float32).astype(np.float64)
    T = 2 * d
    k = np.concatenate([keys, np.zeros((d, d))])
    v = np.concatenate([vals, np.zeros((d, dv))])
    q = np.concatenate([np.zeros((d, d)), keys])
    beta = np.concatenate([np.ones(d), np.zeros(d)])
    out, _ = run1(oracle_lib, None, q, k, v, np.ones((T, d)), beta)
    assert np.array_equal(out[d:], vals)


# --- Decode entry and gate summary ----------------------------------------------

def test_decode_matches_forward(oracle_lib):
    """Stacked single-token steps are the same recurrence as the forward."""
    rng = np.random.default_rng(41)
    B, H, T, Dk, Dv = 2, 3, 12, 6, 4
    q = rng.standard_normal((B, T, H, Dk)); k = rng.standard_normal((B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv)); a = rng.uniform(-1, 1, (B, T, H, Dk))
    b = rng.uniform(0, 2, (B, T, H)); S0 = rng.standard_normal((B, H, Dk, Dv))
    o_f, s_f = oracle_lib.forward(q, k, v, a, b, S0)
    sw = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1))
    o_d, s_d = oracle_lib.decode(sw(q), sw(k), sw(v), sw(a), sw(b), S0.astype(np.float32))
    assert np.allclose(sw(o_d), o_f, rtol=1e-13, atol=1e-13)
    assert np.allclose(s_d, s_f, rtol=1e-13, atol=1e-13)


def test_gate_summary(oracle_lib):
    """[zpos == 0] * (-1)^parity * 2^L equals the plain product of gates from
    the chunk start, for every token, including exact zeros and -1 entries; the
    worked gate [0.9, 0.2] gives L = log2 of its powers."""
    rng = np.random.default_rng(43)
    B, T, H, Dk, C = 1, 37, 2, 5, 16
    a = rng.uniform(-1, 1, (B, T, H, Dk)).astype(np.float32)
    a[rng.random(a.shape) < 0.1] = 0.0
    a[rng.random(a.shape) < 0.1] = -1.0
    g = oracle_lib.gate_prep(a, C)
    NC = (T + C - 1) // C
    for n in range(NC):
        t0 = n * C
        for r in range(min(C, T - t0)):
            prod = np.prod(a[0, t0:t0 + r + 1].astype(np.float64), axis=0)     # [H, Dk]
            rec = (g["zpos"][0, :, n, r] == 0) * np.where(g["parity"][0, :, n, r] == 1, -1.0, 1.0) \
                * np.exp2(g["L"][0, :, n, r])
            assert np.allclose(rec, prod, rtol=1e-12, atol=0)
        last = min(C, T - t0) - 1
        assert np.allclose(g["gend"][0, :, n], np.prod(a[0, t0:t0 + last + 1].astype(np.float64), axis=0))
    w = oracle_lib.gate_prep(np.tile(np.array([0.9, 0.2], np.float32), (1, 3, 1, 1)), 4)
    assert np.allclose(w["L"][0, 0, 0, :3], [[math.log2(0.9 ** t), math.log2(0.2 ** t)] for t in (1, 2, 3)])


def test_gate_summary_ratios(oracle_lib):
    """The decay between any two tokens of a chunk, prod_{j=i+1..r} alpha_j, is
    0 when a zero gate lies in (i, r] (zpos_r > i + 1) and otherwise
    (-1)^(parity_r - parity_i) * 2^(L_r - L_i): the exact-sign, exact-zero form
    of the chunk decay ratios."""
    rng = np.random.default_rng(47)
    T, Dk, C = 32, 6, 32
    a = rng.uniform(-1, 1, (1, T, 1, Dk)).astype(np.float32)
    a[rng.random(a.shape) < 0.08] = 0.0
    a[rng.random(a.shape) < 0.08] = -1.0
    g = oracle_lib.gate_prep(a, C)
    L, par, zp = g["L"][0, 0, 0], g["parity"][0, 0, 0].astype(int), g["zpos"][0, 0, 0]
    for r in range(T):
        for i in range(r):
            prod = np.prod(a[0, i + 1:r + 1, 0].astype(np.float64), axis=0)
            rec = np.where(zp[r] > i + 1, 0.0,
                           np.where((par[r] - par[i]) % 2 == 1, -1.0, 1.0) * np.exp2(L[r] - L[i]))
            assert np.allclose(rec, prod, rtol=1e-12, atol=0)


def test_chunk_start_states_are_prefix_states(oracle_lib):
    """Chunk-start states (the state entering each chunk of the chunkwise form):
    entry 0 is the initial state exactly, and entry n equals the final state of
    the same recurrence run on the first n*chunk tokens only; a recording
    before/after the wrong token, in the wrong slot or for the wrong (b, h)
    breaks the equality.  CKDA gates with exact zeros and -1, beta up to 2,
    a ragged last chunk and B, H > 1."""
    rng = np.random.default_rng(11)
    B, T, H, Dk, Dv, chunk = 2, 29, 3, 8, 5, 8
    q = rng.standard_normal((B, T, H, Dk)).astype(np.float32) * 0.5
    k = rng.standard_normal((B, T, H, Dk)).astype(np.float32) * 0.5
    v = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    a = rng.uniform(-1, 1, (B, T, H, Dk)).astype(np.float32)
    a[0, 3, 1, 2] = 0.0
    a[1, 17, 0, 5] = -1.0
    b = rng.uniform(0, 2, (B, T, H)).astype(np.float32)
    S0 = rng.standard_normal((B, H, Dk, Dv)).astype(np.float32)
    out, ST, CS = oracle_lib.forward(q, k, v, a, b, S0, chunk=chunk)
    NC = (T + chunk - 1) // chunk
    assert CS.shape == (B, H, NC, Dk, Dv)
    assert np.array_equal(CS[:, :, 0], S0.astype(np.float64))
    for n in range(1, NC):
        t = n * chunk
        _, S_pre = oracle_lib.forward(q[:, :t], k[:, :t], v[:, :t], a[:, :t], b[:, :t], S0)
        assert np.array_equal(CS[:, :, n], S_pre), n
    # the outputs and final state do not depend on whether states are recorded
    out2, ST2 = oracle_lib.forward(q, k, v, a, b, S0)
    assert np.array_equal(out, out2) and np.array_equal(ST, ST2)
    # zero initial state: entry 0 is zero
    _, _, CS0 = oracle_lib.forward(q, k, v, a, b, None, chunk=chunk)
    assert not CS0[:, :, 0].any()


def _raw_inputs(seed, B=1, T=23, H=2, Dk=8, Dv=5, unit=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk)).astype(np.float32) * 1.7
    k = rng.standard_normal((B, T, H, Dk)).astype(np.float32) * 0.6
    if unit:
        q = (q / np.linalg.norm(q.astype(np.float64), axis=-1, keepdims=True)).astype(np.float32)
        k = (k / np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    g = (rng.standard_normal((B, T, H, Dk)) * 2).astype(np.float32)
    c = rng.standard_normal((B, T, H)).astype(np.float32)
    S0 = (rng.standard_normal((B, H, Dk, Dv)) * 0.3).astype(np.float32)
    return q, k, v, g, c, S0


def test_prologue_degenerate_gate_range_and_zero_logit_beta(oracle_lib):
    """Eq. (15) with alpha_min = alpha_max = 0.75 gives alpha = 0.75 for any
    logit; eq. (17) at logit 0 gives beta = beta_max / 2 = 1; unit-norm q, k
    pass eq. (18) unchanged (eps = 0).  Must equal the plain recurrence with
    those constants."""
    q, k, v, g, c, S0 = _raw_inputs(3, unit=True)
    c[:] = 0.0
    o, s = oracle_lib.forward_prologue(q, k, v, g, c, S0, alpha_min=0.75, alpha_max=0.75,
                                       beta_max=2.0, eps=0.0, normalize_q=True)
    o_ref, s_ref = oracle_lib.forward(q, k, v, np.full_like(g, 0.75), np.ones_like(c), S0)
    assert np.abs(o - o_ref).max() < 1e-6 and np.abs(s - s_ref).max() < 1e-6


def test_prologue_gate_midpoint_forgets(oracle_lib):
    """Gate logits 0 with the CKDA range [-1, 1] give alpha = 0 exactly (the
    midpoint of eq. (15)), so every token forgets the state: S_t = beta k v^T
    and o_t = beta (q.k) v_t with the normalised q, k, i.e. beta times the
    cosine similarity of the raw vectors (eps = 0, beta logit 0, beta_max 2
    -> beta = 1)."""
    q, k, v, g, c, S0 = _raw_inputs(4)
    g[:] = 0.0
    c[:] = 0.0
    o, s = oracle_lib.forward_prologue(q, k, v, g, c, S0, alpha_min=-1.0, alpha_max=1.0,
                                       beta_max=2.0, eps=0.0, normalize_q=True)
    q64, k64 = q.astype(np.float64), k.astype(np.float64)
    cos = (q64 * k64).sum(-1) / (np.linalg.norm(q64, axis=-1) * np.linalg.norm(k64, axis=-1))
    assert np.abs(o - cos[..., None] * v).max() < 1e-12
    kn = k64[:, -1] / np.linalg.norm(k64[:, -1], axis=-1, keepdims=True)
    assert np.abs(s - kn[..., :, None] * v[:, -1][..., None, :]).max() < 1e-12


def test_prologue_scale_invariance(oracle_lib):
    """Eq. (18) with eps = 0 makes the result independent of the scale of k_raw
    (and of q_raw when q is normalised); without q normalisation the output
    scales with q_raw."""
    q, k, v, g, c, S0 = _raw_inputs(5)
    kw = dict(alpha_min=0.0, alpha_max=1.0, beta_max=1.0, eps=0.0)
    o1, s1 = oracle_lib.forward_prologue(q, k, v, g, c, S0, normalize_q=True, **kw)
    o2, s2 = oracle_lib.forward_prologue(q * 0.25, k * 4.0, v, g, c, S0, normalize_q=True, **kw)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(s1 - s2).max() < 1e-12
    o3, _ = oracle_lib.forward_prologue(q, k, v, g, c, S0, normalize_q=False, **kw)
    o4, _ = oracle_lib.forward_prologue(q * 0.25, k * 4.0, v, g, c, S0, normalize_q=False, **kw)
    assert np.abs(o4 - 0.25 * o3).max() < 1e-12
    assert np.abs(o3 - o1).max() > 1e-3          # q normalisation does something here


def test_prologue_gate_symmetry_and_limits(oracle_lib):
    """sigmoid(-x) = 1 - sigmoid(x): eq. (15) with the range reversed and the
    logits negated gives the same gates; logits of +-40 reach the range ends
    (alpha = alpha_max, or alpha_min) to double precision."""
    q, k, v, g, c, S0 = _raw_inputs(6)
    kw = dict(beta_max=2.0, eps=1e-3, normalize_q=True)
    o1, s1 = oracle_lib.forward_prologue(q, k, v, g, c, S0, alpha_min=-0.5, alpha_max=0.9, **kw)
    o2, s2 = oracle_lib.forward_prologue(q, k, v, -g, c, S0, alpha_min=0.9, alpha_max=-0.5, **kw)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(s1 - s2).max() < 1e-12
    # limits: the same run with gate logits +40 and with alpha fixed at the range end
    hi = np.full_like(g, 40.0)
    o_hi, _ = oracle_lib.forward_prologue(q, k, v, hi, c, S0, alpha_min=-0.5, alpha_max=0.9, **kw)
    o_end, _ = oracle_lib.forward_prologue(q, k, v, g, c, S0, alpha_min=0.9, alpha_max=0.9, **kw)
    assert np.abs(o_hi - o_end).max() < 1e-12
    o_lo, _ = oracle_lib.forward_prologue(q, k, v, -hi, c, S0, alpha_min=-0.5, alpha_max=0.9, **kw)
    o_end2, _ = oracle_lib.forward_prologue(q, k, v, g, c, S0, alpha_min=-0.5, alpha_max=-0.5, **kw)
    assert np.abs(o_lo - o_end2).max() < 1e-12


def _phase_inputs(seed, B=1, T=19, H=2, Dk=8, Dv=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk)).astype(np.float32) * 0.5
    k = rng.standard_normal((B, T, H, Dk)).astype(np.float32) * 0.5
    v = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    a = rng.uniform(0.5, 1.0, (B, T, H, Dk // 2)).astype(np.float32)
    th = rng.uniform(-3.0, 3.0, (B, T, H, Dk // 2)).astype(np.float32)
    b = rng.uniform(0, 1, (B, T, H)).astype(np.float32)
    S0 = rng.standard_normal((B, H, Dk, Dv)).astype(np.float32)
    return q, k, v, a, th, b, S0


def test_phase_zero_is_kda(oracle_lib):
    """Phase variant with theta = 0 is KDA with each pair's decay on both of its
    channels ("Semidirect Fourier Delta Attention", Prop. 2.1)."""
    q, k, v, a, th, b, S0 = _phase_inputs(21)
    o1, s1 = oracle_lib.forward_phase(q, k, v, a, np.zeros_like(th), b, S0)
    o2, s2 = oracle_lib.forward(q, k, v, np.repeat(a, 2, axis=-1), b, S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_phase_beta_zero_is_diagonal_ssm(oracle_lib):
    """beta = 0 leaves S_t = Lambda_t S_{t-1} (Prop. 2.1): per pair, the product
    of the decays times the rotation by the summed phases (rotations of the
    plane compose by adding angles), applied to S0; o_t = S_t^T q_t."""
    q, k, v, a, th, b, S0 = _phase_inputs(22)
    b[:] = 0.0
    o, s = oracle_lib.forward_phase(q, k, v, a, th, b, S0)
    B, T, H, Dk = q.shape
    for t in range(T):
        amp = np.prod(a[:, :t + 1].astype(np.float64), axis=1)         # [B,H,Dk/2]
        ang = np.sum(th[:, :t + 1].astype(np.float64), axis=1)
        S = np.empty(S0.shape, dtype=np.float64)
        x, y = S0[:, :, 0::2].astype(np.float64), S0[:, :, 1::2].astype(np.float64)
        c, sn = (amp * np.cos(ang))[..., None], (amp * np.sin(ang))[..., None]
        S[:, :, 0::2] = c * x - sn * y
        S[:, :, 1::2] = sn * x + c * y
        o_exp = np.einsum("bhkv,bhk->bhv", S, q[:, t].astype(np.float64))
        assert np.abs(o[:, t] - o_exp).max() < 1e-12
    assert np.abs(s - S).max() < 1e-12


def test_phase_pi_is_negative_gate(oracle_lib):
    """theta = pi turns each pair's block into -alpha I: the same recurrence as
    the gate -alpha on both channels (the CKDA range).  The phases are fp32, so
    pi carries a sine of about 9e-8; the bound allows for that."""
    q, k, v, a, th, b, S0 = _phase_inputs(23)
    o1, s1 = oracle_lib.forward_phase(q, k, v, a, np.full_like(th, np.pi), b, S0)
    o2, s2 = oracle_lib.forward(q, k, v, -np.repeat(a, 2, axis=-1), b, S0)
    assert np.abs(o1 - o2).max() < 1e-5 and np.abs(s1 - s2).max() < 1e-5
    # ... while theta = 0 against the gate -alpha differs at order one
    o3, _ = oracle_lib.forward_phase(q, k, v, a, np.zeros_like(th), b, S0)
    assert np.abs(o3 - o2).max() > 1e-2


def test_phase_rotation_preserves_norm(oracle_lib):
    """alpha = 1, beta = 0: every step is a rotation of each row pair, so the
    Frobenius norm of the state never changes."""
    q, k, v, a, th, b, S0 = _phase_inputs(24, T=40)
    a[:] = 1.0
    b[:] = 0.0
    for T in (1, 7, 40):
        _, s = oracle_lib.forward_phase(q[:, :T], k[:, :T], v[:, :T], a[:, :T], th[:, :T],
                                        b[:, :T], S0)
        n0 = np.sqrt((S0.astype(np.float64) ** 2).sum(axis=(-2, -1)))
        n1 = np.sqrt((s ** 2).sum(axis=(-2, -1)))
        assert np.abs(n1 - n0).max() < 1e-12 * n0.max()


def test_prologue_eps_sits_outside_the_norm(oracle_lib):
    """Eq. (18) ("Semidirect Fourier Delta Attention", §3) adds eps to the norm
    itself: k = k_raw / (|k_raw|_2 + eps).  One token with the gate range
    collapsed to {0} (eq. (15) with alpha_min = alpha_max = 0: the state is
    forgotten) and beta = 2 sigmoid(0) = 1 (eq. (17)) leaves S_1 = k v^T, so
    the normalised key is read off the state.  k_raw = (3, 4, 0, ...) has norm
    5; with eps = 1 the key is k_raw / 6 exactly, while eps under the root
    (sqrt(25 + 1)) or squared (sqrt(25) + 1 with eps^2, the same here) is told
    apart by a second eps = 2 case: k_raw / 7, not k_raw / sqrt(29) or / 9.
    With q normalised the same way, q_raw = (6, 8, 0, ...) (norm 10) gives
    o_1 = (q.k) v with q.k = (3 6 + 4 8) / (6 11) = 50 / 66."""
    Dk, Dv = 8, 3
    q = np.zeros((1, 1, 1, Dk), np.float32)
    k = np.zeros((1, 1, 1, Dk), np.float32)
    q[..., 0], q[..., 1] = 6.0, 8.0
    k[..., 0], k[..., 1] = 3.0, 4.0
    v = np.array([1.5, -2.0, 0.25], np.float32).reshape(1, 1, 1, Dv)
    g = np.full((1, 1, 1, Dk), 0.7, np.float32)          # any logit: the range is {0}
    c = np.zeros((1, 1, 1), np.float32)
    S0 = np.full((1, 1, Dk, Dv), 3.0, np.float32)        # forgotten by alpha = 0
    v64 = v.reshape(Dv).astype(np.float64)
    for eps, kden, qden in ((1.0, 6.0, 11.0), (2.0, 7.0, 12.0), (0.5, 5.5, 10.5)):
        o, s = oracle_lib.forward_prologue(q, k, v, g, c, S0, alpha_min=0.0, alpha_max=0.0,
                                           beta_max=2.0, eps=eps, normalize_q=True)
        kn = np.zeros(Dk)
        kn[0], kn[1] = 3.0 / kden, 4.0 / kden
        assert np.abs(s[0, 0] - np.outer(kn, v64)).max() < 1e-15, eps
        qk = (3.0 * 6.0 + 4.0 * 8.0) / (kden * qden)
        assert np.abs(o[0, 0, 0] - qk * v64).max() < 1e-15, eps
        # without q normalisation the raw q reads the same state
        o2, _ = oracle_lib.forward_prologue(q, k, v, g, c, S0, alpha_min=0.0, alpha_max=0.0,
                                            beta_max=2.0, eps=eps, normalize_q=False)
        assert np.abs(o2[0, 0, 0] - (50.0 / kden) * v64).max() < 1e-14, eps
