"""Pins for the fp64 oracle (CPU only).

Each test fixes the oracle to something other than itself: a hand-worked
example, a closed form, an invariant the pages state, or a special case that
reduces to a textbook identity.  A plausible slip in the recurrence (a
dropped erase term, a wrong sign, the decay applied after the prediction, a
transposed state, the read taken before the write) fails at least one.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import (
    gated_delta_recurrence,
    recurrent_step,
    additive_closed_form,
    unrolled_transition_sum,
    scalar_recurrence_d1,
    chunked_gated_delta,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand_inputs(rng, B, T, H, Dk, Dv, gate, s0=False, beta_scale=1.0):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    beta = beta_scale / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    if gate == "none":
        la = None
    elif gate == "scalar":
        la = -np.log1p(np.exp(rng.normal(-2.0, 0.5, (B, T, H))))
    else:
        la = -np.log1p(np.exp(rng.normal(-3.0, 1.0, (B, T, H, Dk))))
    S0 = rng.standard_normal((B, H, Dk, Dv)) * 0.3 if s0 else None
    return q, k, v, beta, la, S0


# ---------------------------------------------------------------------------
# hand-worked examples


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"],
                         ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    q = np.array(case["q"], float)[None, :, None, :]
    k = np.array(case["k"], float)[None, :, None, :]
    v = np.array(case["v"], float)[None, :, None, :]
    beta = np.array(case["beta"], float)[None, :, None]
    if case["alpha"] is None:
        la = None
    else:
        a = np.log(np.array(case["alpha"], float))
        la = a[None, :, None] if a.ndim == 1 else a[None, :, None, :]
    S0 = np.array(case["S0"], float)[None, None]
    o, S = gated_delta_recurrence(q, k, v, beta, la, S0)
    np.testing.assert_allclose(o[0, :, 0], np.array(case["o"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(S[0, 0], np.array(case["S_T"]), rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# P1: exact recall with orthonormal keys (the orthogonal-key capacity
# argument of linear attention, and the delta rule's overwrite behaviour)


def _orthonormal(rng, d, n):
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return Qm[:, :n].T  # n orthonormal rows


def test_exact_recall_and_overwrite():
    rng = np.random.default_rng(1)
    d, n = 8, 6
    keys = _orthonormal(rng, d, n)
    vals = rng.standard_normal((n, 5))
    # write all n pairs, then read each key back; then overwrite key 2
    T = n + n + 1 + 1
    k = np.zeros((1, T, 1, d)); q = np.zeros((1, T, 1, d))
    v = np.zeros((1, T, 1, 5)); beta = np.zeros((1, T, 1))
    for i in range(n):
        k[0, i, 0] = keys[i]; v[0, i, 0] = vals[i]; beta[0, i, 0] = 1.0
        q[0, i, 0] = keys[0]
    for i in range(n):  # read-only steps (beta = 0), query key i
        k[0, n + i, 0] = keys[i]; q[0, n + i, 0] = keys[i]
    new_val = rng.standard_normal(5)
    k[0, 2 * n, 0] = keys[2]; v[0, 2 * n, 0] = new_val; beta[0, 2 * n, 0] = 1.0
    q[0, 2 * n, 0] = keys[2]
    k[0, 2 * n + 1, 0] = keys[3]; q[0, 2 * n + 1, 0] = keys[3]
    o, _ = gated_delta_recurrence(q, k, v, beta)
    for i in range(n):
        np.testing.assert_allclose(o[0, n + i, 0], vals[i], atol=1e-12)
        # the read at write step i with query key 0 already sees key 0's value
        np.testing.assert_allclose(o[0, i, 0], vals[0], atol=1e-12)
    np.testing.assert_allclose(o[0, 2 * n, 0], new_val, atol=1e-12)      # overwritten
    np.testing.assert_allclose(o[0, 2 * n + 1, 0], vals[3], atol=1e-12)  # untouched
    # additive linear attention instead accumulates: old + new
    o_add, _ = gated_delta_recurrence(q, k, v, beta, erase=False)
    np.testing.assert_allclose(o_add[0, 2 * n, 0], vals[2] + new_val, atol=1e-12)


# ---------------------------------------------------------------------------
# P1': beta_t = 1 and |k_t| = 1 make the step an exact projection: the new
# memory returns v_t for k_t, whatever the history and the gate.


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_one_step_recall_invariant(gate):
    rng = np.random.default_rng(2)
    q, k, v, beta, la, S0 = _rand_inputs(rng, 2, 9, 3, 7, 4, gate, s0=True)
    t = 6
    beta[:, t] = 1.0
    q[:, t] = k[:, t]
    o, _ = gated_delta_recurrence(q, k, v, beta, la, S0)
    np.testing.assert_allclose(o[:, t], v[:, t], atol=1e-12)
    # with beta < 1 it must NOT hold (guards against an ignored beta)
    beta[:, t] = 0.5
    o2, _ = gated_delta_recurrence(q, k, v, beta, la, S0)
    assert np.max(np.abs(o2[:, t] - v[:, t])) > 1e-3


# ---------------------------------------------------------------------------
# P2: additive closed forms


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_additive_switch_matches_closed_form(gate):
    rng = np.random.default_rng(3)
    q, k, v, beta, la, _ = _rand_inputs(rng, 2, 11, 2, 5, 3, gate)
    o, _ = gated_delta_recurrence(q, k, v, beta, la, erase=False)
    ref = additive_closed_form(q, k, v, beta, la)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_plain_linear_attention_closed_form():
    # alpha = beta = 1, no erase: o_t = sum_{s<=t} (q_t . k_s) v_s
    rng = np.random.default_rng(4)
    q, k, v, _, _, _ = _rand_inputs(rng, 1, 13, 2, 6, 4, "none")
    beta = np.ones((1, 13, 2))
    o, _ = gated_delta_recurrence(q, k, v, beta, erase=False)
    ref = np.zeros_like(o)
    for t in range(13):
        for s in range(t + 1):
            ref[:, t] += np.sum(q[:, t] * k[:, s], -1)[..., None] * v[:, s]
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_delta_rule_with_orthogonal_keys_is_additive_scalar_gate():
    # k_t^T S_{t-1} = 0 for mutually orthogonal keys, so the erase term is
    # identically zero and the delta rule writes beta_s v_s additively.
    rng = np.random.default_rng(5)
    d, T = 10, 8
    keys = _orthonormal(rng, d, T)
    q, _, v, beta, la, _ = _rand_inputs(rng, 1, T, 1, d, 3, "scalar")
    k = keys[None, :, None, :]
    o, _ = gated_delta_recurrence(q, k, v, beta, la)
    ref = additive_closed_form(q, k, v, beta, la)
    np.testing.assert_allclose(o, ref, atol=1e-12)
    # with non-orthogonal keys they differ
    q2, k2, v2, b2, la2, _ = _rand_inputs(rng, 1, T, 1, d, 3, "scalar")
    o2, _ = gated_delta_recurrence(q2, k2, v2, b2, la2)
    assert np.max(np.abs(o2 - additive_closed_form(q2, k2, v2, b2, la2))) > 1e-3


def test_delta_rule_with_axis_keys_is_additive_channel_gate():
    # per-channel decay keeps standard-basis keys orthogonal after scaling
    rng = np.random.default_rng(6)
    d, T = 9, 7
    perm = rng.permutation(d)[:T]
    k = np.zeros((1, T, 1, d))
    for t in range(T):
        k[0, t, 0, perm[t]] = rng.choice([-1.0, 1.0])
    q, _, v, beta, la, _ = _rand_inputs(rng, 1, T, 1, d, 4, "channel")
    o, _ = gated_delta_recurrence(q, k, v, beta, la)
    np.testing.assert_allclose(o, additive_closed_form(q, k, v, beta, la), atol=1e-12)


# ---------------------------------------------------------------------------
# P3: the chunkwise (WY / triangular solve) form equals the recurrence


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("T,chunk", [(1, 1), (1, 16), (5, 2), (16, 16), (37, 4),
                                     (37, 16), (37, 64), (70, 16), (70, 64), (64, 64)])
def test_chunked_equals_recurrence(gate, T, chunk):
    rng = np.random.default_rng(7 + T + chunk)
    q, k, v, beta, la, S0 = _rand_inputs(rng, 2, T, 2, 8, 5, gate, s0=True)
    o, S = gated_delta_recurrence(q, k, v, beta, la, S0)
    oc, Sc = chunked_gated_delta(q, k, v, beta, la, S0, chunk=chunk)
    np.testing.assert_allclose(oc, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(Sc, S, atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# P4: KDA with every channel equal to the scalar decay is GDN


def test_channel_gate_with_equal_channels_is_scalar_gate():
    rng = np.random.default_rng(8)
    q, k, v, beta, la, S0 = _rand_inputs(rng, 2, 15, 3, 6, 4, "scalar", s0=True)
    la_c = np.repeat(la[..., None], 6, axis=-1)
    o1, S1 = gated_delta_recurrence(q, k, v, beta, la, S0)
    o2, S2 = gated_delta_recurrence(q, k, v, beta, la_c, S0)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(S2, S1, atol=1e-13)
    # but KDA is not GDN in general (the decay applies to rows of S)
    la_r = la_c + rng.normal(0, 0.3, la_c.shape)
    o3, _ = gated_delta_recurrence(q, k, v, beta, np.minimum(la_r, 0), S0)
    assert np.max(np.abs(o3 - o1)) > 1e-3


def test_kda_decays_rows_before_erasing():
    # decay-then-erase (I - b k k^T) Diag(a) S differs from erase-then-decay
    rng = np.random.default_rng(9)
    q, k, v, beta, la, S0 = _rand_inputs(rng, 1, 1, 1, 4, 3, "channel", s0=True)
    o, S = gated_delta_recurrence(q, k, v, beta, la, S0)
    a = np.exp(la[0, 0, 0]); kk = k[0, 0, 0]; b = beta[0, 0, 0]
    E = np.eye(4) - b * np.outer(kk, kk)
    want = E @ np.diag(a) @ S0[0, 0] + b * np.outer(kk, v[0, 0, 0])
    other = np.diag(a) @ E @ S0[0, 0] + b * np.outer(kk, v[0, 0, 0])
    np.testing.assert_allclose(S[0, 0], want, atol=1e-13)
    assert np.max(np.abs(want - other)) > 1e-4


# ---------------------------------------------------------------------------
# P5: special cases


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_zero_beta_only_decays(gate):
    rng = np.random.default_rng(10)
    q, k, v, beta, la, S0 = _rand_inputs(rng, 2, 12, 2, 5, 3, gate, s0=True)
    beta[:] = 0.0
    o, S = gated_delta_recurrence(q, k, v, beta, la, S0)
    if gate == "none":
        g = np.zeros((2, 12, 2, 5))
    elif gate == "scalar":
        g = np.repeat(np.cumsum(la, axis=1)[..., None], 5, axis=-1)
    else:
        g = np.cumsum(la, axis=1)
    for t in range(12):
        St = np.exp(g[:, t])[..., None] * S0            # Diag(e^{g_t}) S0
        np.testing.assert_allclose(o[:, t], np.einsum("bhkv,bhk->bhv", St, q[:, t]), atol=1e-12)
    np.testing.assert_allclose(S, np.exp(g[:, -1])[..., None] * S0, atol=1e-12)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_hard_reset_gate(gate):
    # log alpha = -50 wipes the memory: o_t = beta_t (k_t . q_t) v_t, no NaN
    rng = np.random.default_rng(11)
    q, k, v, beta, la, S0 = _rand_inputs(rng, 1, 6, 2, 5, 3, gate, s0=True)
    la[:] = -50.0
    o, S = gated_delta_recurrence(q, k, v, beta, la, S0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    want = (beta * np.sum(k * q, -1))[..., None] * v
    np.testing.assert_allclose(o, want, atol=1e-15)


def test_single_token_closed_form():
    rng = np.random.default_rng(12)
    q, k, v, beta, la, S0 = _rand_inputs(rng, 1, 1, 1, 6, 4, "scalar", s0=True)
    o, S = gated_delta_recurrence(q, k, v, beta, la, S0)
    a = math.exp(la[0, 0, 0]); kk = k[0, 0, 0]; b = beta[0, 0, 0]
    S1 = a * (np.eye(6) - b * np.outer(kk, kk)) @ S0[0, 0] + b * np.outer(kk, v[0, 0, 0])
    np.testing.assert_allclose(S[0, 0], S1, atol=1e-13)
    np.testing.assert_allclose(o[0, 0, 0], S1.T @ q[0, 0, 0], atol=1e-13)


def test_scalar_case_by_hand():
    rng = np.random.default_rng(13)
    T = 25
    qs, ks, vs = rng.standard_normal(T), rng.standard_normal(T), rng.standard_normal(T)
    bs = rng.uniform(0, 1, T)
    las = -rng.uniform(0, 1, T)
    out, s = scalar_recurrence_d1(qs, ks, vs, bs, np.exp(las), s0=0.7)
    o, S = gated_delta_recurrence(qs.reshape(1, T, 1, 1), ks.reshape(1, T, 1, 1),
                                  vs.reshape(1, T, 1, 1), bs.reshape(1, T, 1),
                                  las.reshape(1, T, 1), np.full((1, 1, 1, 1), 0.7))
    np.testing.assert_allclose(o[0, :, 0, 0], out, atol=1e-13)
    assert abs(S[0, 0, 0, 0] - s) < 1e-13


# ---------------------------------------------------------------------------
# P6: state passing (the memory is the whole carry: split anywhere, resume)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_state_passing(gate):
    rng = np.random.default_rng(14)
    q, k, v, beta, la, S0 = _rand_inputs(rng, 2, 20, 2, 6, 4, gate, s0=True)
    o, S = gated_delta_recurrence(q, k, v, beta, la, S0)
    for t0 in (1, 7, 19):
        cut = lambda x, a, b: None if x is None else x[:, a:b]
        o1, S1 = gated_delta_recurrence(q[:, :t0], k[:, :t0], v[:, :t0], beta[:, :t0],
                                        cut(la, 0, t0), S0)
        o2, S2 = gated_delta_recurrence(q[:, t0:], k[:, t0:], v[:, t0:], beta[:, t0:],
                                        cut(la, t0, None), S1)
        np.testing.assert_allclose(np.concatenate([o1, o2], 1), o, atol=1e-13)
        np.testing.assert_allclose(S2, S, atol=1e-13)
    # the decode-step form is the same recurrence one token at a time
    St = S0.copy()
    for t in range(20):
        ot, St = recurrent_step(q[:, t], k[:, t], v[:, t], beta[:, t],
                                None if la is None else la[:, t], St)
        np.testing.assert_allclose(ot, o[:, t], atol=1e-13)
    np.testing.assert_allclose(St, S, atol=1e-13)


# ---------------------------------------------------------------------------
# P7: explicit transition-matrix products (the unrolled form)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_unrolled_transition_products(gate):
    rng = np.random.default_rng(15)
    q, k, v, beta, la, S0 = _rand_inputs(rng, 1, 7, 2, 4, 3, gate, s0=True)
    o, S = gated_delta_recurrence(q, k, v, beta, la, S0)
    ou, Su = unrolled_transition_sum(q, k, v, beta, la, S0)
    np.testing.assert_allclose(ou, o, atol=1e-12)
    np.testing.assert_allclose(Su, S, atol=1e-12)


# ---------------------------------------------------------------------------
# P8: linearity in (V, S_0) for fixed keys and gates, and in q


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_linearity(gate):
    rng = np.random.default_rng(16)
    q, k, v, beta, la, S0 = _rand_inputs(rng, 1, 10, 2, 5, 3, gate, s0=True)
    _, _, v2, _, _, S02 = _rand_inputs(rng, 1, 10, 2, 5, 3, gate, s0=True)
    a, b = 0.7, -1.3
    o1, S1 = gated_delta_recurrence(q, k, v, beta, la, S0)
    o2, S2 = gated_delta_recurrence(q, k, v2, beta, la, S02)
    o3, S3 = gated_delta_recurrence(q, k, a * v + b * v2, beta, la, a * S0 + b * S02)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-12)
    np.testing.assert_allclose(S3, a * S1 + b * S2, atol=1e-12)
    q2 = rng.standard_normal(q.shape)
    o4, _ = gated_delta_recurrence(q2, k, v, beta, la, S0)
    o5, _ = gated_delta_recurrence(a * q + b * q2, k, v, beta, la, S0)
    np.testing.assert_allclose(o5, a * o1 + b * o4, atol=1e-12)
