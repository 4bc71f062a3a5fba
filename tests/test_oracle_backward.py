"""Pins of the backward oracle (CPU only).

The backward oracle is checked against something other than itself:
- central finite differences of L = <dout, out> computed by the forward
  oracle (itself pinned in test_oracle_pins.py), for every element of every
  input array, in both conv modes, with and without the residual, at several
  conv widths;
- the table-row gradient against a dense scatter-add (numpy.add.at) over
  whole tables;
- a special case with a closed form: gamma_k = 0 makes the gate constant 1/2,
  so no gradient reaches W_k and the hidden state gets exactly dout back.
"""

import numpy as np
import pytest

import oracle


def _layer_arrays(rng, Br, d, De, batch, seqlen, kc):
    n_tok = batch * seqlen
    return {
        "emb": rng.standard_normal((n_tok, De)).astype(np.float32),
        "h": rng.standard_normal((Br, n_tok, d)).astype(np.float32),
        "w_k": (rng.standard_normal((Br, d, De)) / np.sqrt(De)).astype(np.float32),
        "w_v": (rng.standard_normal((d, De)) / np.sqrt(De)).astype(np.float32),
        "gamma_h": (1.0 + 0.1 * rng.standard_normal((Br, d))).astype(np.float32),
        "gamma_k": (1.0 + 0.1 * rng.standard_normal((Br, d))).astype(np.float32),
        "conv_w": (0.5 * rng.standard_normal((d, kc))).astype(np.float32),
    }


def _loss(a, dout, batch, seqlen, mode, flags):
    L = oracle.Layer(a["emb"], a["h"], a["w_k"], a["w_v"], a["gamma_h"], a["gamma_k"], a["conv_w"],
                     batch, seqlen, oracle.F32, conv_mode=mode, flags=flags)
    out, _, _ = L.forward_all()
    return float(np.sum(out * dout))


GRAD_OF = {"emb": "demb", "h": "dh", "w_k": "dw_k", "w_v": "dw_v", "gamma_h": "dgamma_h",
           "gamma_k": "dgamma_k", "conv_w": "dconv_w"}


@pytest.mark.parametrize("mode,flags,kc", [(oracle.CONV_LINEAR, 0, 3), (oracle.CONV_SILU_SKIP, 0, 4),
                                           (oracle.CONV_LINEAR, oracle.OUT_DELTA, 1),
                                           (oracle.CONV_SILU_SKIP, oracle.OUT_DELTA, 2)])
def test_backward_matches_finite_differences(mode, flags, kc):
    rng = np.random.default_rng(100 + 10 * mode + kc)
    Br, d, De, batch, seqlen = 2, 8, 12, 2, 6
    a = _layer_arrays(rng, Br, d, De, batch, seqlen, kc)
    dout = rng.standard_normal((Br, batch * seqlen, d)).astype(np.float32)
    L = oracle.Layer(a["emb"], a["h"], a["w_k"], a["w_v"], a["gamma_h"], a["gamma_k"], a["conv_w"],
                     batch, seqlen, oracle.F32, conv_mode=mode, flags=flags)
    g = L.backward(dout)
    for name, gname in GRAD_OF.items():
        x = a[name]
        an = g[gname].reshape(x.shape)
        scale = float(np.sqrt(np.mean(an ** 2))) + 1e-12
        fd = np.zeros_like(an)
        for i in np.ndindex(x.shape):
            x0 = x[i]
            step = np.float32(1e-3 * max(abs(float(x0)), float(np.sqrt(np.mean(x.astype(np.float64) ** 2)))))
            xp, xm = np.float32(x0 + step), np.float32(x0 - step)
            x[i] = xp
            lp = _loss(a, dout, batch, seqlen, mode, flags)
            x[i] = xm
            lm = _loss(a, dout, batch, seqlen, mode, flags)
            x[i] = x0
            fd[i] = (lp - lm) / (float(xp) - float(xm))
        err = np.abs(fd - an) / (np.abs(an) + scale)
        assert err.max() < 2e-4, (name, float(err.max()), np.unravel_index(np.argmax(err), err.shape))


def test_constant_gate_sends_no_gradient_to_w_k():
    rng = np.random.default_rng(7)
    Br, d, De, batch, seqlen, kc = 1, 8, 12, 2, 5, 3
    a = _layer_arrays(rng, Br, d, De, batch, seqlen, kc)
    a["gamma_k"][:] = 0.0
    dout = rng.standard_normal((Br, batch * seqlen, d)).astype(np.float32)
    L = oracle.Layer(a["emb"], a["h"], a["w_k"], a["w_v"], a["gamma_h"], a["gamma_k"], a["conv_w"],
                     batch, seqlen, oracle.F32)
    g = L.backward(dout)
    assert np.all(g["dw_k"] == 0.0) and np.all(g["dgamma_h"] == 0.0)
    assert np.array_equal(g["dh"], dout.astype(np.float64))


@pytest.mark.parametrize("n_tok,n_tables,rows_per_table,head_dim", [(1, 1, 7, 4), (50, 3, 5, 8), (300, 4, 97, 6)])
def test_table_grad_equals_dense_scatter_add(n_tok, n_tables, rows_per_table, head_dim):
    rng = np.random.default_rng(n_tok)
    idx = rng.integers(0, rows_per_table, (n_tok, n_tables)).astype(np.uint32)
    demb = rng.standard_normal((n_tok, n_tables * head_dim))
    rows, grads, counts = oracle.table_grad(idx, demb, head_dim)
    for tau in range(n_tables):
        dense = np.zeros((rows_per_table, head_dim))
        np.add.at(dense, idx[:, tau].astype(np.int64), demb[:, tau * head_dim:(tau + 1) * head_dim])
        used = np.unique(idx[:, tau])
        assert counts[tau] == len(used)
        assert np.array_equal(rows[tau, :counts[tau]], used)
        np.testing.assert_allclose(grads[tau, :counts[tau]], dense[used], rtol=1e-12, atol=1e-12)
