"""The chunk-wise algebra the GPU kernels implement reproduces the token
recurrence of the oracle (float64, no kernels involved)."""
import numpy as np

import oracle
from tests import chunked_ref as CR
from tests.test_oracle_pins import rand_inputs


def test_chunked_forward_equals_token_oracle():
    rng = np.random.default_rng(21)
    q, k, v, g, s, beta = rand_inputs(rng, 2, 150, 16, 8, p_neg=0.3)
    S0 = rng.standard_normal((2, 16, 8))
    o, ST = oracle.fwd_chain_arrays(q, k, v, g, s, beta, 0.8, S0)
    for i in range(2):
        for anchored in (False, True):
            oc, Sc = CR.fwd_chain(q[i], k[i], v[i], g[i], s[i], beta[i], 0.8, S0[i], anchored=anchored)
            np.testing.assert_allclose(oc, o[i], rtol=0, atol=1e-12)
            np.testing.assert_allclose(Sc, ST[i], rtol=0, atol=1e-12)


def test_record_form_equals_token_oracle():
    """The split forward: a state-independent record per chunk, then the
    state pass U = u - W S, O = Qh S + M U, S <- Diag(d) S + KbT U."""
    rng = np.random.default_rng(24)
    q, k, v, g, s, beta = rand_inputs(rng, 2, 150, 16, 8, p_neg=0.3)
    S0 = rng.standard_normal((2, 16, 8))
    o, ST = oracle.fwd_chain_arrays(q, k, v, g, s, beta, 0.8, S0)
    for i in range(2):
        oc, Sc = CR.fwd_chain_record(q[i], k[i], v[i], g[i], s[i], beta[i], 0.8, S0[i])
        np.testing.assert_allclose(oc, o[i], rtol=0, atol=1e-12)
        np.testing.assert_allclose(Sc, ST[i], rtol=0, atol=1e-12)


def test_chunked_backward_equals_token_oracle():
    rng = np.random.default_rng(22)
    q, k, v, g, s, beta = rand_inputs(rng, 1, 140, 8, 6, p_neg=0.3)
    S0 = rng.standard_normal((1, 8, 6))
    do = rng.standard_normal((1, 140, 6))
    dST = rng.standard_normal((1, 8, 6))
    r = oracle.bwd_chain_arrays(q, k, v, g, s, beta, do, 1.2, S0, dST)
    rc = CR.bwd_chain(q[0], k[0], v[0], g[0], s[0], beta[0], do[0], 1.2, S0[0], dST[0])
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        ref = r[name][0]
        np.testing.assert_allclose(rc[name], ref, rtol=0, atol=1e-11 * (1 + np.abs(ref).max()),
                                   err_msg=name)


def test_anchored_chunked_backward_equals_token_oracle():
    rng = np.random.default_rng(23)
    q, k, v, g, s, beta = rand_inputs(rng, 1, 150, 8, 6, p_neg=0.3)
    S0 = rng.standard_normal((1, 8, 6))
    do = rng.standard_normal((1, 150, 6))
    dST = rng.standard_normal((1, 8, 6))
    r = oracle.bwd_chain_arrays(q, k, v, g, s, beta, do, 0.9, S0, dST)
    rc = CR.bwd_chain_anchored(q[0], k[0], v[0], g[0], s[0], beta[0], do[0], 0.9, S0[0], dST[0])
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        ref = r[name][0]
        np.testing.assert_allclose(rc[name], ref, rtol=0, atol=1e-11 * (1 + np.abs(ref).max()),
                                   err_msg=name)
