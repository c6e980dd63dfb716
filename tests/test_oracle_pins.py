"""Pins of the fp64 CPU oracle to facts outside itself.

The Ling & Ring 2.6 Technical Report pages print no operator values, so the
oracle is pinned by mathematics: a worked example derived by hand from the
definition, the quadratic (masked-matrix) form, closed-form special cases,
linearity, continuation of the state, the context-parallel state algebra the
pages describe ("Context Parallel for Lightning Attention": local recursion plus
a global correction) and central finite differences for the backward.  Packed
(varlen) batches are pinned to the block-diagonal masked-matrix form, to
prefix caching (continuing from a cached state) and to the independence of
the sequences.  The output epilogue (gated group RMSNorm) is pinned to a
hand-computed example, closed-form properties and scipy's logistic function.
"""
import numpy as np
import pytest

import la_inputs


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _relerr(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- worked example
# H=1, N=3, d=2.  q0=(1,0) q1=(0,1) q2=(1,2); k0=(1,1) k1=(2,-1) k2=(0,1);
# v0=(1,2) v1=(-1,0) v2=(3,1); dO0=(1,-1) dO1=(2,1) dO2=(0,1).
# By hand from o_t = sum_{s<=t} lam^(t-s) (q_t.k_s) v_s:
#   q.k:  q0k0=1; q1k0=1, q1k1=-1; q2k0=3, q2k1=0, q2k2=2
#   o0 = 1*v0                         = (1, 2)
#   o1 = lam*1*v0 + (-1)*v1           = (lam+1, 2lam)
#   o2 = 3lam^2 v0 + 0*v1 + 2 v2      = (3lam^2+6, 6lam^2+2)
#   S2 = lam^2 k0v0^T + lam k1v1^T + k2v2^T
#      = [[lam^2-2lam, 2lam^2], [lam^2+lam+3, 2lam^2+1]]
# Backward of L = sum_t o_t.dO_t:
#   dq_t = S_t dO_t with S0=[[1,2],[1,2]], S1=[[lam-2,2lam],[lam+1,2lam]]:
#     dq0=(-1,-1), dq1=(4lam-4, 4lam+2), dq2=(2lam^2, 2lam^2+1)
#   dk_s = sum_{t>=s} lam^(t-s) (dO_t.v_s) q_t, with dO.v: d0v0=-1, d1v0=4, d2v0=2,
#     d1v1=-2, d2v1=0, d2v2=1:
#     dk0 = -q0 + 4lam q1 + 2lam^2 q2 = (2lam^2-1, 4lam^2+4lam); dk1=(0,-2); dk2=(1,2)
#   dv_s = sum_{t>=s} lam^(t-s) (q_t.k_s) dO_t:
#     dv0 = dO0 + lam dO1 + 3lam^2 dO2 = (1+2lam, 3lam^2+lam-1); dv1=(-2,-1); dv2=(0,2)
_WQ = [[1, 0], [0, 1], [1, 2]]
_WK = [[1, 1], [2, -1], [0, 1]]
_WV = [[1, 2], [-1, 0], [3, 1]]
_WG = [[1, -1], [2, 1], [0, 1]]


def _worked_expected(lam):
    L = lam
    o = [[1, 2], [L + 1, 2 * L], [3 * L**2 + 6, 6 * L**2 + 2]]
    S2 = [[L**2 - 2 * L, 2 * L**2], [L**2 + L + 3, 2 * L**2 + 1]]
    dq = [[-1, -1], [4 * L - 4, 4 * L + 2], [2 * L**2, 2 * L**2 + 1]]
    dk = [[2 * L**2 - 1, 4 * L**2 + 4 * L], [0, -2], [1, 2]]
    dv = [[1 + 2 * L, 3 * L**2 + L - 1], [-2, -1], [0, 2]]
    return [np.array(x, dtype=np.float64) for x in (o, S2, dq, dk, dv)]


@pytest.mark.parametrize("slope", [0.0, 0.3, 1.7])
def test_worked_example_by_hand(oracle_mod, slope):
    s = np.array([slope], dtype=np.float32)
    lam = np.exp(-np.float64(s[0]))
    q, k, v, g = (np.array(x, dtype=np.float64)[None, None] for x in (_WQ, _WK, _WV, _WG))
    o, S = oracle_mod.fwd(q, k, v, s)
    dq, dk, dv = oracle_mod.bwd(q, k, v, g, s)
    eo, eS, edq, edk, edv = _worked_expected(lam)
    np.testing.assert_allclose(o[0, 0], eo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S[0, 0], eS, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dq[0, 0], edq, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk[0, 0], edk, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv[0, 0], edv, rtol=0, atol=1e-13)
    # the quadratic form agrees with the same hand values
    bo, bS = oracle_mod.brute.fwd(q, k, v, s)
    np.testing.assert_allclose(bo[0, 0], eo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(bS[0, 0], eS, rtol=0, atol=1e-13)


# ----------------------------------------------------------- quadratic vs recurrent
@pytest.mark.parametrize("with_s0", [False, True])
def test_recurrent_matches_quadratic(oracle_mod, with_s0):
    rng = _rng(11)
    B, H, N, d = 2, 3, 37, 8
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    s = np.array([0.05, 0.7, 2.5], dtype=np.float32)
    S0 = _rand(rng, B, H, d, d) if with_s0 else None
    o, S = oracle_mod.fwd(q, k, v, s, S0)
    bo, bS = oracle_mod.brute.fwd(q, k, v, s, S0)
    assert _relerr(o, bo) < 1e-12
    assert _relerr(S, bS) < 1e-12


@pytest.mark.parametrize("C", [1, 4, 16, 64, 256])
def test_chunked_matches_recurrent(oracle_mod, C):
    rng = _rng(12)
    B, H, N, d = 1, 4, 100, 16
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    s = la_inputs.slopes(H)
    S0 = _rand(rng, B, H, d, d)
    o, S = oracle_mod.fwd(q, k, v, s, S0)
    co, cS = oracle_mod.fwd_chunked(q, k, v, s, C, S0)
    assert _relerr(co, o) < 1e-12
    assert _relerr(cS, S) < 1e-12


# ------------------------------------------------------------------ special cases
def test_no_decay_is_plain_causal_linear_attention(oracle_mod):
    # slope 0 -> lambda 1: S_t is the running sum of k v^T (numpy cumsum).
    rng = _rng(13)
    B, H, N, d = 1, 2, 20, 5
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    s = np.zeros(H, dtype=np.float32)
    o, S = oracle_mod.fwd(q, k, v, s)
    outer = np.einsum("bhti,bhtj->bhtij", k, v)
    St = np.cumsum(outer, axis=2)
    eo = np.einsum("bhti,bhtij->bhtj", q, St)
    assert _relerr(o, eo) < 1e-13
    assert _relerr(S, St[:, :, -1]) < 1e-13


def test_full_decay_keeps_only_the_current_token(oracle_mod):
    # exp(-1e4) == 0 in fp64, so o_t = (q_t . k_t) v_t and S_N = k_{N-1} v_{N-1}^T
    rng = _rng(14)
    B, H, N, d = 2, 1, 9, 4
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    s = np.array([1.0e4], dtype=np.float32)
    o, S = oracle_mod.fwd(q, k, v, s, _rand(rng, B, H, d, d))
    eo = np.sum(q * k, axis=-1, keepdims=True) * v
    np.testing.assert_allclose(o, eo, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(S, np.einsum("bhi,bhj->bhij", k[:, :, -1], v[:, :, -1]), rtol=1e-14, atol=1e-14)


def test_single_token(oracle_mod):
    rng = _rng(15)
    B, H, d = 1, 2, 6
    q, k, v = (_rand(rng, B, H, 1, d) for _ in range(3))
    S0 = _rand(rng, B, H, d, d)
    s = np.array([0.25, 1.5], dtype=np.float32)
    lam = np.exp(-s.astype(np.float64))
    o, S = oracle_mod.fwd(q, k, v, s, S0)
    for h in range(H):
        qh, kh, vh = q[0, h, 0], k[0, h, 0], v[0, h, 0]
        np.testing.assert_allclose(o[0, h, 0], (qh @ kh) * vh + lam[h] * (qh @ S0[0, h]), rtol=1e-13)
        np.testing.assert_allclose(S[0, h], np.outer(kh, vh) + lam[h] * S0[0, h], rtol=1e-13)


def test_linearity(oracle_mod):
    rng = _rng(16)
    B, H, N, d = 1, 2, 15, 4
    q1, q2, k, v1, v2 = (_rand(rng, B, H, N, d) for _ in range(5))
    s = np.array([0.1, 0.9], dtype=np.float32)
    oa, _ = oracle_mod.fwd(q1 + q2, k, v1, s)
    ob, _ = oracle_mod.fwd(q1, k, v1, s)
    oc, _ = oracle_mod.fwd(q2, k, v1, s)
    assert _relerr(oa, ob + oc) < 1e-13
    od, Sd = oracle_mod.fwd(q1, k, 3.0 * v1 - 2.0 * v2, s)
    oe, Se = oracle_mod.fwd(q1, k, v1, s)
    of, Sf = oracle_mod.fwd(q1, k, v2, s)
    assert _relerr(od, 3 * oe - 2 * of) < 1e-13
    assert _relerr(Sd, 3 * Se - 2 * Sf) < 1e-13
    og, Sg = oracle_mod.fwd(q1, -0.5 * k, v1, s)
    assert _relerr(og, -0.5 * oe) < 1e-13 and _relerr(Sg, -0.5 * Se) < 1e-13


def test_continuation_of_the_state(oracle_mod):
    rng = _rng(17)
    B, H, N1, N2, d = 2, 2, 23, 18, 6
    q, k, v = (_rand(rng, B, H, N1 + N2, d) for _ in range(3))
    s = np.array([0.02, 0.6], dtype=np.float32)
    o, S = oracle_mod.fwd(q, k, v, s)
    o1, S1 = oracle_mod.fwd(q[:, :, :N1], k[:, :, :N1], v[:, :, :N1], s)
    o2, S2 = oracle_mod.fwd(q[:, :, N1:], k[:, :, N1:], v[:, :, N1:], s, S1)
    assert _relerr(np.concatenate([o1, o2], axis=2), o) < 1e-13
    assert _relerr(S2, S) < 1e-13


def test_decode_steps_equal_prefill(oracle_mod):
    rng = _rng(18)
    B, H, N, d = 3, 2, 12, 5
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    S0 = _rand(rng, B, H, d, d, scale=0.1)
    s = np.array([0.3, 0.01], dtype=np.float32)
    o, S = oracle_mod.fwd(q, k, v, s, S0)
    st = S0
    for t in range(N):
        ot, st = oracle_mod.decode(q[:, :, t], k[:, :, t], v[:, :, t], s, st)
        np.testing.assert_allclose(ot, o[:, :, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, S, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("bounds", [(0, 40, 90, 130), (0, 1, 2, 130), (0, 64, 128)])
def test_context_parallel_state_algebra(oracle_mod, bounds):
    """Local recursion per shard from a zero state, then a global correction.

    For shard r = [t_r, t_{r+1}): S_in(r) = sum_{r'<r} lambda^(t_r - t_{r'+1}) S_loc(r'),
    and o_t = o_loc_t + lambda^(t - t_r + 1) q_t^T S_in(r)."""
    rng = _rng(19)
    B, H, d = 1, 3, 4
    N = bounds[-1]
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    s = np.array([0.003, 0.05, 0.4], dtype=np.float32)
    lam = np.exp(-s.astype(np.float64))
    o, S = oracle_mod.fwd(q, k, v, s)
    locs = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        locs.append(oracle_mod.fwd(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], s))
    corrected = []
    for r, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        S_in = np.zeros((B, H, d, d))
        for rp in range(r):
            end = bounds[rp + 1]
            S_in += (lam ** (a - end))[None, :, None, None] * locs[rp][1]
        t = np.arange(a, b)
        fac = lam[None, :, None] ** (t - a + 1)[None, None, :]
        corr = fac[..., None] * np.einsum("bhti,bhij->bhtj", q[:, :, a:b], S_in)
        corrected.append(locs[r][0] + corr)
    assert _relerr(np.concatenate(corrected, axis=2), o) < 1e-12


# ------------------------------------------------------------ packed sequences
_CU_CASES = [(0, 7, 7, 8, 30, 61), (0, 61), (0, 1, 2, 3), (0, 0, 20)]


def _packed(seed, H, T, d):
    rng = _rng(seed)
    return tuple(_rand(rng, H, T, d) for _ in range(3))


@pytest.mark.parametrize("cu", _CU_CASES)
@pytest.mark.parametrize("with_s0", [False, True])
def test_varlen_matches_packed_quadratic_form(oracle_mod, cu, with_s0):
    """Recurrence per sequence against the block-diagonal masked-matrix form."""
    H, d = 2, 5
    q, k, v = _packed(30, H, cu[-1], d)
    S0 = _rand(_rng(31), len(cu) - 1, H, d, d) if with_s0 else None
    s = np.array([0.05, 0.9], dtype=np.float32)
    o, S = oracle_mod.fwd_varlen(q, k, v, s, cu, S0)
    ob, Sb = oracle_mod.brute.fwd_varlen(q, k, v, s, cu, S0)
    assert _relerr(o, ob) < 1e-12 and _relerr(S, Sb) < 1e-12


def test_packed_quadratic_form_with_one_sequence_is_the_plain_form(oracle_mod):
    H, T, d = 3, 19, 4
    q, k, v = _packed(32, H, T, d)
    S0 = _rand(_rng(33), 1, H, d, d)
    s = np.array([0.0, 0.2, 2.0], dtype=np.float32)
    o, S = oracle_mod.brute.fwd_varlen(q, k, v, s, (0, T), S0)
    op, Sp = oracle_mod.brute.fwd(q[None], k[None], v[None], s, S0)
    assert _relerr(o, op[0]) < 1e-13 and _relerr(S, Sp) < 1e-13


def test_varlen_prefix_caching(oracle_mod):
    """A sequence continued from the cached state of its prefix gives the
    outputs and final state of the whole sequence."""
    H, T, m, d = 2, 45, 17, 6
    q, k, v = _packed(34, H, T, d)
    S0 = _rand(_rng(35), 1, H, d, d, scale=0.3)
    s = np.array([0.01, 0.4], dtype=np.float32)
    o, S = oracle_mod.fwd_varlen(q, k, v, s, (0, T), S0)
    o1, S1 = oracle_mod.fwd_varlen(q[:, :m], k[:, :m], v[:, :m], s, (0, m), S0)
    o2, S2 = oracle_mod.fwd_varlen(q[:, m:], k[:, m:], v[:, m:], s, (0, T - m), S1)
    assert _relerr(np.concatenate([o1, o2], axis=1), o) < 1e-13
    assert _relerr(S2, S) < 1e-13


def test_varlen_sequences_are_independent(oracle_mod):
    cu = (0, 11, 11, 30, 42)
    H, d = 2, 4
    q, k, v = _packed(36, H, cu[-1], d)
    s = np.array([0.0, 0.3], dtype=np.float32)
    o, S = oracle_mod.fwd_varlen(q, k, v, s, cu)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[:, 11:30] += 1.0  # sequence 2 only
    o2, S2 = oracle_mod.fwd_varlen(q2, k2, v2, s, cu)
    keep = np.r_[0:11, 30:42]
    assert np.array_equal(o[:, keep], o2[:, keep])
    assert np.array_equal(S[[0, 1, 3]], S2[[0, 1, 3]])
    assert not np.allclose(o[:, 11:30], o2[:, 11:30])
    # the empty sequence passes its (zero) initial state through
    assert np.array_equal(S[1], np.zeros_like(S[1]))


@pytest.mark.parametrize("cu", _CU_CASES)
def test_varlen_backward_matches_packed_quadratic_form(oracle_mod, cu):
    H, d = 2, 5
    q, k, v = _packed(37, H, cu[-1], d)
    g = _rand(_rng(38), H, cu[-1], d)
    s = np.array([0.05, 0.9], dtype=np.float32)
    got = oracle_mod.bwd_varlen(q, k, v, g, s, cu)
    ref = oracle_mod.brute.bwd_varlen(q, k, v, g, s, cu)
    for a, b in zip(got, ref):
        if b.size:
            assert _relerr(a, b) < 1e-12


def test_varlen_backward_finite_differences(oracle_mod):
    """Central differences of L = sum(o * dO) through the packed forward."""
    cu = (0, 9, 10, 33)
    H, d = 2, 4
    q, k, v = _packed(39, H, cu[-1], d)
    g = _rand(_rng(40), H, cu[-1], d)
    s = np.array([0.1, 0.7], dtype=np.float32)
    grads = oracle_mod.bwd_varlen(q, k, v, g, s, cu)
    eps = 1e-6
    rng = _rng(41)
    for which in range(3):
        for _ in range(40):
            ix = tuple(rng.integers(0, n) for n in q.shape)
            xs = [q.copy(), k.copy(), v.copy()]
            xs[which][ix] += eps
            lp = np.sum(oracle_mod.fwd_varlen(*xs, s, cu)[0] * g)
            xs[which][ix] -= 2 * eps
            lm = np.sum(oracle_mod.fwd_varlen(*xs, s, cu)[0] * g)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grads[which][ix]) < 1e-6 * max(1.0, np.max(np.abs(grads[which])))


# ------------------------------------------------------------- output epilogue
def test_gated_norm_worked_example(oracle_mod):
    """By hand, one token of one head, d = 2: o = (3, 4) has mean square
    12.5; with eps = 0, weight (1, 2) and gate (0, ln 3):
    y = (3, 4) / sqrt(12.5) * (1, 2) * (1/2, 3/4) = (0.42426..., 1.69705...)."""
    o = np.array([[[[3.0, 4.0]]]])
    g = np.array([[[[0.0, np.log(3.0)]]]])
    w = np.array([[1.0, 2.0]])
    y = oracle_mod.gated_group_rmsnorm(o, g, w, 0.0)
    r = np.sqrt(12.5)
    np.testing.assert_allclose(y[0, 0, 0], [3 / r * 0.5, 4 / r * 2 * 0.75], rtol=1e-15)


def test_gated_norm_properties(oracle_mod):
    rng = _rng(50)
    B, H, N, d = 2, 3, 7, 16
    o = _rand(rng, B, H, N, d)
    g = _rand(rng, B, H, N, d, scale=2.0)
    w = _rand(rng, H, d)
    eps = 1e-5
    y = oracle_mod.gated_group_rmsnorm(o, g, w, eps)
    # a huge gate passes the normalised row through: unit RMS up to eps
    big = np.full_like(g, 60.0)
    yu = oracle_mod.gated_group_rmsnorm(o, big, np.ones((H, d)), eps)
    ms = np.mean(o * o, axis=-1)
    np.testing.assert_allclose(np.mean(yu * yu, axis=-1), ms / (ms + eps), rtol=1e-12)
    # gate 0 halves it
    y0 = oracle_mod.gated_group_rmsnorm(o, np.zeros_like(g), np.ones((H, d)), eps)
    np.testing.assert_allclose(y0, 0.5 * yu, rtol=1e-12)
    # with eps = 0 the result is invariant to scaling a row by c > 0 and odd in o
    y1 = oracle_mod.gated_group_rmsnorm(o, g, w, 0.0)
    y2 = oracle_mod.gated_group_rmsnorm(-7.5 * o, g, w, 0.0)
    np.testing.assert_allclose(y2, -y1, rtol=1e-12)
    # the gate is the logistic function (scipy's expit), the weight per (head, channel)
    from scipy.special import expit
    h, j = 2, 5
    ref = o[..., h, :, j] / np.sqrt(np.mean(o[..., h, :, :] ** 2, axis=-1) + eps) * w[h, j] * expit(g[..., h, :, j])
    np.testing.assert_allclose(y[..., h, :, j], ref, rtol=1e-12)


def test_fwd_gated_composes(oracle_mod):
    rng = _rng(51)
    B, H, N, d = 1, 2, 20, 8
    q, k, v, g = (_rand(rng, B, H, N, d) for _ in range(4))
    w = _rand(rng, H, d)
    s = np.array([0.1, 0.5], dtype=np.float32)
    y, S = oracle_mod.fwd_gated(q, k, v, s, g, w, 1e-6)
    ob, Sb = oracle_mod.brute.fwd(q, k, v, s)
    ms = np.mean(ob * ob, axis=-1, keepdims=True)
    assert _relerr(y, ob / np.sqrt(ms + 1e-6) * w[:, None, :] / (1 + np.exp(-g))) < 1e-12
    assert _relerr(S, Sb) < 1e-12


# ---------------------------------------------------------------------- backward
def test_backward_matches_quadratic_closed_form(oracle_mod):
    rng = _rng(20)
    B, H, N, d = 2, 2, 33, 8
    q, k, v, g = (_rand(rng, B, H, N, d) for _ in range(4))
    S0 = _rand(rng, B, H, d, d)
    s = np.array([0.08, 1.1], dtype=np.float32)
    got = oracle_mod.bwd(q, k, v, g, s, S0)
    ref = oracle_mod.brute.bwd(q, k, v, g, s, S0)
    for a, b in zip(got, ref):
        assert _relerr(a, b) < 1e-12


def test_backward_finite_differences(oracle_mod):
    """Central differences of L = sum(o * dO) on the B=1, H=2, N=64, d=16 instance."""
    B, H, N, d = 1, 2, 64, 16
    q, k, v = la_inputs.qkv(4, B, H, N, d, dtype="f32")
    g = la_inputs.upstream_grad(4, B, H, N, d, dtype="f32")
    q, k, v, g = (x.astype(np.float64) for x in (q, k, v, g))
    s = la_inputs.slopes(H)
    dq, dk, dv = oracle_mod.bwd(q, k, v, g, s)
    eps = 1e-6
    rng = _rng(21)
    for name, grad, which in (("q", dq, 0), ("k", dk, 1), ("v", dv, 2)):
        idx = [tuple(rng.integers(0, n) for n in (B, H, N, d)) for _ in range(300)]
        fd = np.empty(len(idx))
        an = np.empty(len(idx))
        for m, ix in enumerate(idx):
            xs = [q.copy(), k.copy(), v.copy()]
            xs[which][ix] += eps
            lp = np.sum(oracle_mod.fwd(*xs, s)[0] * g)
            xs[which][ix] -= 2 * eps
            lm = np.sum(oracle_mod.fwd(*xs, s)[0] * g)
            fd[m] = (lp - lm) / (2 * eps)
            an[m] = grad[ix]
        err = np.max(np.abs(fd - an)) / np.max(np.abs(an))
        assert err < 1e-6, (name, err)


# ------------------------------------------------------------------ input recipe
def test_slopes_follow_the_geometric_recipe():
    for H in (2, 16, 32):
        s = la_inputs.slopes(H).astype(np.float64)
        assert s[-1] == 2.0**-8  # h = H-1 gives exactly 2^(-8)
        np.testing.assert_allclose(s[1:] / s[:-1], 2.0 ** (-8.0 / H), rtol=1e-6)
        np.testing.assert_allclose(s[0], 2.0 ** (-8.0 / H), rtol=1e-7)
    lam = np.exp(-la_inputs.slopes(32).astype(np.float64))
    assert abs(lam[0] - 0.4313) < 1e-4 and abs(lam[31] - 0.99610) < 1e-5


def test_bf16_rounding_matches_torch():
    import torch

    rng = _rng(22)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-30, 30, 100000)).astype(np.float32)
    x[:4] = [1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8), 0.0]
    ours = la_inputs.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)
    assert ours[0] == 1.0 and ours[1] == 1.0 + 2.0**-6


def test_frozen_tiny_workload(oracle_mod):
    """Regression guard: oracle output on the tiny fp32 workload is unchanged."""
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny_f32.json")
    with open(path) as f:
        ref = json.load(f)
    c = la_inputs.CONFIGS["tiny_f32"]
    q, k, v = la_inputs.qkv(c["seed"], c["B"], c["H"], c["N"], c["d"], dtype="f32")
    o, S = oracle_mod.fwd(q, k, v, la_inputs.slopes(c["H"]))
    for h in range(c["H"]):
        np.testing.assert_allclose(o[0, h, ref["rows"]], np.array(ref["o_rows"][str(h)]), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(np.diag(S[0, h]), np.array(ref["S_diag"][str(h)]), rtol=1e-12, atol=1e-14)
        assert abs(S[0, h].sum() - ref["S_sum"][h]) < 1e-10
