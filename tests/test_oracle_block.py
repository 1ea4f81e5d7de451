"""Pins for the Mamba-2 block's short convolution and gated RMS norm oracle.

* The causal convolution equals numpy.convolve per channel (a library
  routine) with the kernel reversed, before the SiLU; an impulse reads the
  weights back newest-last; the decode form (last W-1 inputs) equals the
  whole-sequence form; drafts and a commit of k equal stepping the k accepted
  inputs.
* The gated norm equals torch's rms_norm (a library routine) over each group
  of the gated values; with weight 1 every group has unit RMS; a large
  positive gate reduces it to the plain RMS norm of y.
"""
import numpy as np
import torch

from oracle import block


def _case(seed, T=12, b=3, C=10, W=4):
    g = np.random.default_rng(seed)
    return g.standard_normal((T, b, C)), g.standard_normal((C, W)), g.standard_normal(C)


def test_conv_equals_numpy_convolve():
    seq, w, bias = _case(1)
    out = block.causal_conv(seq, w, bias)
    T, b, C = seq.shape
    for bb in range(b):
        for c in range(C):
            pre = np.convolve(seq[:, bb, c], w[c][::-1])[:T] + bias[c]
            np.testing.assert_allclose(out[:, bb, c], pre / (1 + np.exp(-pre)), rtol=1e-13, atol=1e-14)


def test_conv_impulse_reads_weights():
    _, w, _ = _case(2)
    T, C, W = 6, w.shape[0], w.shape[1]
    seq = np.zeros((T, 1, C))
    seq[0] = 1.0
    out = block.causal_conv(seq, w)
    for t in range(W):
        np.testing.assert_allclose(out[t, 0], block.silu(w[:, W - 1 - t]), rtol=1e-14)
    assert np.all(out[W:] == 0.0)


def test_decode_form_and_drafts():
    seq, w, bias = _case(3, T=20)
    full = block.causal_conv(seq, w, bias)
    st = block.ConvState(seq.shape[1], seq.shape[2], w, bias)
    for t in range(10):
        np.testing.assert_allclose(st.step(seq[t]), full[t], rtol=1e-13, atol=1e-14)
    drafts = [seq[10 + d] for d in range(4)]
    outs = st.drafts(drafts)
    np.testing.assert_allclose(outs, full[10:14], rtol=1e-13, atol=1e-14)
    st.commit(drafts, np.array([2, 2, 2]))
    np.testing.assert_allclose(st.step(seq[12]), full[12], rtol=1e-13, atol=1e-14)
    # a sequence that accepted only 1 continues from token 11
    st2 = block.ConvState(seq.shape[1], seq.shape[2], w, bias)
    for t in range(10):
        st2.step(seq[t])
    st2.commit(drafts, np.array([1, 3, 0]))
    alt = seq[11].copy()
    alt[0] = seq[11][0]                     # sequence 0: next input is token 11
    alt[1] = seq[13][1]                     # sequence 1: token 13
    alt[2] = seq[10][2]                     # sequence 2: token 10
    o = st2.step(alt)
    np.testing.assert_allclose(o[0], full[11][0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o[1], full[13][1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o[2], full[10][2], rtol=1e-13, atol=1e-14)


def test_gated_norm_equals_torch_rms_norm():
    g = np.random.default_rng(4)
    b, d, ng = 3, 64, 4
    y, z, wt = g.standard_normal((b, d)), g.standard_normal((b, d)), g.standard_normal(d)
    out = block.gated_rmsnorm(y, z, wt, ng, eps=1e-5)
    v = torch.from_numpy(y * (z / (1 + np.exp(-z)))).view(b, ng, d // ng)
    ref = torch.nn.functional.rms_norm(v, (d // ng,), eps=1e-5).reshape(b, d).numpy() * wt
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    unit = block.gated_rmsnorm(y, z, np.ones(d), ng, eps=0.0).reshape(b, ng, d // ng)
    np.testing.assert_allclose(np.sqrt(np.mean(unit ** 2, axis=-1)), 1.0, rtol=1e-12)
    open_gate = block.gated_rmsnorm(y, np.full((b, d), 40.0), np.ones(d), ng, eps=0.0)
    yy = y.reshape(b, ng, d // ng)
    plain = (yy / np.sqrt(np.mean(yy ** 2, axis=-1, keepdims=True))).reshape(b, d)
    np.testing.assert_allclose(open_gate, plain, rtol=1e-12)
