"""Pins of the backward oracle (oracle/backward.py): every gradient against
central finite differences of the forward recurrence oracle, for every gate,
with and without the erase term, with an initial state and a loss that
weights both the outputs and the final state."""

import numpy as np
import pytest

from oracle import gated_delta_backward, gated_delta_recurrence


def _inputs(gate, seed, B=1, T=5, H=2, Dk=3, Dv=2):
    rng = np.random.default_rng(seed)
    inp = {
        "q": rng.normal(size=(B, T, H, Dk)),
        "k": rng.normal(size=(B, T, H, Dk)) * 0.6,
        "v": rng.normal(size=(B, T, H, Dv)),
        "beta": rng.uniform(0.2, 0.9, size=(B, T, H)),
        "log_alpha": None,
        "initial_state": rng.normal(size=(B, H, Dk, Dv)) * 0.5,
    }
    if gate == "scalar":
        inp["log_alpha"] = rng.uniform(-0.8, -0.05, size=(B, T, H))
    elif gate == "channel":
        inp["log_alpha"] = rng.uniform(-0.8, -0.05, size=(B, T, H, Dk))
    w_o = rng.normal(size=(B, T, H, Dv))
    w_s = rng.normal(size=(B, H, Dk, Dv))
    return inp, w_o, w_s


def _loss(inp, w_o, w_s, erase):
    o, S = gated_delta_recurrence(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                                  inp["initial_state"], erase=erase)
    return float(np.sum(o * w_o) + np.sum(S * w_s))


def _fd(inp, name, w_o, w_s, erase, h=1e-6):
    x = inp[name]
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        old = x[idx]
        x[idx] = old + h
        lp = _loss(inp, w_o, w_s, erase)
        x[idx] = old - h
        lm = _loss(inp, w_o, w_s, erase)
        x[idx] = old
        g[idx] = (lp - lm) / (2 * h)
    return g


@pytest.mark.parametrize("erase", [True, False])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_gradients_match_finite_differences(gate, erase):
    inp, w_o, w_s = _inputs(gate, seed=len(gate) + 10 * erase)
    got = gated_delta_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                               inp["initial_state"], d_o=w_o, d_final=w_s, erase=erase)
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"),
             ("initial_state", "dS0")]
    if gate != "none":
        names.append(("log_alpha", "dlog_alpha"))
    for name, gname in names:
        want = _fd(inp, name, w_o, w_s, erase)
        np.testing.assert_allclose(got[gname], want, rtol=1e-6, atol=1e-7, err_msg=gname)
    if gate == "none":
        assert got["dlog_alpha"] is None


def test_zero_loss_gradient_gives_zero_gradients():
    inp, _, _ = _inputs("channel", seed=3)
    got = gated_delta_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                               inp["initial_state"])
    for key, val in got.items():
        assert np.all(val == 0.0), key


def test_output_gradient_only_reaches_the_past():
    # dL/do at the last token only: nothing changes the gradients of q at
    # earlier tokens (o_t reads S_t, which later tokens do not touch)
    inp, w_o, _ = _inputs("scalar", seed=5, T=4)
    w_o[:, :-1] = 0.0
    got = gated_delta_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                               inp["initial_state"], d_o=w_o)
    assert np.all(got["dq"][:, :-1] == 0.0)
    assert np.any(got["dq"][:, -1] != 0.0)
