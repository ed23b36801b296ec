"""Recorded-graph autograd (tt_graph_*) against the oracle.

* the tiny classifier — Linear(3->32) -> tanh-GELU -> Linear(32->4) -> mean
  cross-entropy -> SGD lr 0.1 — recorded once, then five training steps
  through forward / zero_grad / backward / tt_sgd_step, each against
  oracle.mlp_step on the previous step's oracle weights;
* a node used twice (its gradient is the sum of both uses), leaf gradients
  accumulating over two backward calls, and zero_grad;
* a softmax node inside the graph (oracle.softmax_bwd), and a forward of a
  sub-graph after the input changed (inference on the trained weights);
* a deeper chain at shapes spanning several GEMM tiles with ragged tails;
* host-side validation errors;
* the step captured as one HIP graph, replayed five times, each replay
  checked against the eager step and the oracle.
"""

import numpy as np
import pytest

import oracle
from oracle import gpt2 as og
import autograd_transformer_amd as tt
from autograd_transformer_amd import synthetic as syn
from tests.conftest import rel_l2
from tests.gpu_util import dev, host, zeros, sync

pytestmark = pytest.mark.gpu

TOL = 1e-5   # float32 parity bar


@pytest.fixture
def ctx():
    c = tt.Context(arena_bytes=1 << 26)
    yield c
    c.close()


def test_graph_trains_the_tiny_classifier(ctx):
    d = syn.mlp_inputs(seed=1)
    P = {k: dev(d[k]) for k in ("W1", "b1", "W2", "b2")}
    G = {k: zeros(tuple(v.shape)) for k, v in P.items()}
    g = tt.Graph(ctx)
    x = g.leaf(dev(d["x"]))
    ids = {k: g.leaf(P[k], G[k]) for k in P}
    hidden = g.gelu(g.add(g.matmul(x, ids["W1"]), ids["b1"]))
    logits = g.add(g.matmul(hidden, ids["W2"]), ids["b2"])
    loss = g.cross_entropy(logits, dev(d["labels"], "i32"))
    assert g.grad(x) is None
    W = {k: d[k].astype(np.float64) for k in P}
    for step in range(5):
        g.forward(loss)
        g.zero_grad()
        g.backward(loss)
        got_loss = host(g.value(loss))[0, 0]
        got_grads = {k: host(G[k]) for k in P}
        for k in P:
            tt.tt_sgd_step(ctx, P[k], G[k], 0.1)
        sync()
        l_ref, g_ref, new_ref, z_ref = og.mlp_step(d["x"], W["W1"], W["b1"], W["W2"], W["b2"],
                                                   d["labels"])
        assert abs(got_loss - l_ref) <= TOL * abs(l_ref), step
        assert rel_l2(host(g.value(logits)), z_ref) <= TOL, step
        for k in P:
            assert rel_l2(got_grads[k], g_ref[k]) <= TOL, (step, k)
            assert rel_l2(host(P[k]), new_ref[k]) <= TOL, (step, k)
        W = new_ref
    g.close()


def test_graph_shared_node_and_accumulation(ctx):
    rng = np.random.default_rng(5)
    xs, Ws = rng.standard_normal((16, 8)), rng.standard_normal((8, 5))
    y = rng.integers(0, 5, 16)
    Wd, Gd = dev(Ws), zeros((8, 5))
    g = tt.Graph(ctx)
    x, w = g.leaf(dev(xs)), g.leaf(Wd, Gd)
    h = g.matmul(x, w)
    z = g.add(h, h)                      # h feeds one node twice
    loss = g.cross_entropy(z, dev(y, "i32"))
    g.forward(loss)
    g.zero_grad()
    g.backward(loss)
    sync()
    l_ref, dz = oracle.cross_entropy_fwdbwd(2 * (xs @ Ws), y)
    _, dW_ref, _ = oracle.linear_bwd(xs, Ws, 2 * dz, with_bias=False)
    assert abs(host(g.value(loss))[0, 0] - l_ref) <= TOL * l_ref
    assert rel_l2(host(g.grad(h)), 2 * dz) <= TOL
    assert rel_l2(host(Gd), dW_ref) <= TOL
    g.backward(loss)                     # leaf gradients accumulate
    sync()
    assert rel_l2(host(Gd), 2 * dW_ref) <= TOL
    assert rel_l2(host(g.grad(h)), 2 * dz) <= TOL   # interior ones restart
    g.zero_grad()
    sync()
    assert not np.any(host(Gd))
    g.close()


def test_graph_softmax_node_and_partial_forward(ctx):
    rng = np.random.default_rng(6)
    n, k, m, c = 40, 12, 9, 6
    xs = rng.standard_normal((n, k))
    Wa, ba, Wb = rng.standard_normal((k, m)), rng.standard_normal(m), rng.standard_normal((m, c))
    y = rng.integers(0, c, n)
    xd = dev(xs)
    T = {"Wa": dev(Wa), "ba": dev(ba), "Wb": dev(Wb)}
    GT = {kk: zeros(tuple(v.shape)) for kk, v in T.items()}
    g = tt.Graph(ctx)
    x = g.leaf(xd)
    ids = {kk: g.leaf(T[kk], GT[kk]) for kk in T}
    probs = g.softmax(g.add(g.matmul(x, ids["Wa"]), ids["ba"]))
    loss = g.cross_entropy(g.matmul(probs, ids["Wb"]), dev(y, "i32"))
    g.forward(loss)
    g.zero_grad()
    g.backward(loss)
    sync()
    z1 = oracle.linear_fwd(xs, Wa, ba)
    p = oracle.softmax_rows(z1)
    l_ref, dz2 = oracle.cross_entropy_fwdbwd(p @ Wb, y)
    dp, dWb, _ = oracle.linear_bwd(p, Wb, dz2, with_bias=False)
    dz1 = oracle.softmax_bwd(p, dp)
    _, dWa, dba = oracle.linear_bwd(xs, Wa, dz1)
    assert abs(host(g.value(loss))[0, 0] - l_ref) <= TOL * abs(l_ref)
    assert rel_l2(host(g.value(probs)), p) <= TOL
    assert rel_l2(host(GT["Wb"]), dWb) <= TOL
    assert rel_l2(host(GT["Wa"]), dWa) <= TOL
    assert rel_l2(host(GT["ba"]).ravel(), dba) <= TOL
    # new input in place, then only the probabilities (inference)
    xs2 = rng.standard_normal((n, k))
    xd.copy_(dev(xs2))
    g.forward(probs)
    sync()
    assert rel_l2(host(g.value(probs)), oracle.softmax_rows(oracle.linear_fwd(xs2, Wa, ba))) <= TOL
    g.close()


def test_graph_deeper_chain_ragged_shapes(ctx):
    """Shapes spanning several GEMM tiles with ragged tails."""
    rng = np.random.default_rng(7)
    n, d0, d1, c = 300, 70, 131, 45
    xs = rng.standard_normal((n, d0))
    W1, b1 = rng.standard_normal((d0, d1)) * 0.2, rng.standard_normal(d1) * 0.1
    W2, b2 = rng.standard_normal((d1, c)) * 0.2, rng.standard_normal(c) * 0.1
    y = rng.integers(0, c, n)
    T = {"W1": dev(W1), "b1": dev(b1), "W2": dev(W2), "b2": dev(b2)}
    GT = {kk: zeros(tuple(v.shape)) for kk, v in T.items()}
    Gx = zeros((n, d0))
    g = tt.Graph(ctx)
    x = g.leaf(dev(xs), Gx)
    ids = {kk: g.leaf(T[kk], GT[kk]) for kk in T}
    h = g.gelu(g.add(g.matmul(x, ids["W1"]), ids["b1"]))
    loss = g.cross_entropy(g.add(g.matmul(h, ids["W2"]), ids["b2"]), dev(y, "i32"))
    g.forward(loss)
    g.zero_grad()
    g.backward(loss)
    sync()
    hpre = oracle.linear_fwd(xs, W1, b1)
    hh = oracle.gelu_fwd(hpre)
    l_ref, dz = oracle.cross_entropy_fwdbwd(oracle.linear_fwd(hh, W2, b2), y)
    dh, dW2, db2 = oracle.linear_bwd(hh, W2, dz)
    dx, dW1, db1 = oracle.linear_bwd(xs, W1, oracle.gelu_bwd(hpre, dh))
    assert abs(host(g.value(loss))[0, 0] - l_ref) <= TOL * abs(l_ref)
    for got, ref in ((GT["W1"], dW1), (GT["b1"], db1), (GT["W2"], dW2), (GT["b2"], db2),
                     (Gx, dx)):
        assert rel_l2(host(got).ravel(), ref.ravel()) <= TOL
    g.close()


def test_graph_validation_errors(ctx):
    g = tt.Graph(ctx)
    a = g.leaf(zeros((64, 3)))
    b = g.leaf(zeros((4, 32)), zeros((4, 32)))
    with pytest.raises(tt.TTError, match="matmul"):
        g.matmul(a, b)
    with pytest.raises(tt.TTError, match="bad input id"):
        g.gelu(99)
    with pytest.raises(tt.TTError, match="add"):
        g.add(a, b)
    with pytest.raises(tt.TTError, match="loss"):
        g.backward(a)                     # a leaf
    h = g.matmul(g.leaf(zeros((64, 4))), b)
    with pytest.raises(tt.TTError, match="loss"):
        g.backward(h)                     # not [1, 1]
    buf = zeros((65,))
    with pytest.raises(tt.TTError, match="alignment"):
        g.leaf(buf[1:].view(8, 8))
    g.close()
    tt.lib().tt_graph_destroy(None)


def test_captured_step_replays_match_eager_and_oracle(ctx):
    """The tiny classifier's step captured as one HIP graph: five replays,
    each followed by the same step run eagerly on a second copy of the
    weights, and both against the oracle's step."""
    d = syn.mlp_inputs(seed=2)

    def build():
        P = {k: dev(d[k]) for k in ("W1", "b1", "W2", "b2")}
        G = {k: zeros(tuple(v.shape)) for k, v in P.items()}
        g = tt.Graph(ctx)
        x = g.leaf(dev(d["x"]))
        ids = {k: g.leaf(P[k], G[k]) for k in P}
        h = g.gelu(g.add(g.matmul(x, ids["W1"]), ids["b1"]))
        loss = g.cross_entropy(g.add(g.matmul(h, ids["W2"]), ids["b2"]), dev(d["labels"], "i32"))
        return g, P, G, loss

    gc, Pc, Gc, lc = build()
    ge, Pe, Ge, le = build()
    gc.capture_sgd_step(lc, 0.1)
    sync()
    for k in Pc:   # capturing runs nothing
        assert np.array_equal(host(Pc[k]), d[k].astype(np.float64))
    W = {k: d[k].astype(np.float64) for k in Pc}
    for step in range(5):
        gc.step()
        sync()
        got_loss = host(gc.value(lc))[0, 0]
        ge.forward(le)
        ge.zero_grad()
        ge.backward(le)
        for k in Pe:
            tt.tt_sgd_step(ctx, Pe[k], Ge[k], 0.1)
        sync()
        l_ref, g_ref, new_ref, _ = og.mlp_step(d["x"], W["W1"], W["b1"], W["W2"], W["b2"],
                                               d["labels"])
        assert abs(got_loss - host(ge.value(le))[0, 0]) <= 1e-6 * abs(l_ref), step
        assert abs(got_loss - l_ref) <= TOL * abs(l_ref), step
        for k in Pc:
            assert rel_l2(host(Pc[k]), host(Pe[k])) <= 1e-6, (step, k)
            assert rel_l2(host(Gc[k]), g_ref[k]) <= TOL, (step, k)
            assert rel_l2(host(Pc[k]), new_ref[k]) <= TOL, (step, k)
        W = new_ref
    gc.close()
    ge.close()


# ------------------------------------------------ the step as one launch

@pytest.mark.parametrize("N,I,H,C,seed", [(64, 3, 32, 4, 1), (100, 7, 50, 10, 3), (1, 3, 32, 4, 4)])
def test_fused_mlp_step_against_oracle(ctx, N, I, H, C, seed):
    """tt_mlp_step (forward, cross-entropy, backward, SGD in one kernel), five
    steps, each against oracle.mlp_step."""
    d = syn.mlp_inputs(seed=seed, batch=N, n_in=I, hidden=H, classes=C)
    P = {k: dev(d[k]) for k in ("W1", "b1", "W2", "b2")}
    G = {k: zeros(tuple(v.shape)) for k, v in P.items()}
    xd, yd = dev(d["x"]), dev(d["labels"], "i32")
    loss = zeros((1,))
    W = {k: d[k].astype(np.float64) for k in P}
    for step in range(5):
        tt.tt_mlp_step(ctx, xd, yd, P["W1"], P["b1"], P["W2"], P["b2"], 0.1, loss, G)
        sync()
        l_ref, g_ref, new_ref, _ = og.mlp_step(d["x"], W["W1"], W["b1"], W["W2"], W["b2"],
                                               d["labels"])
        # (the N=1 case predicts its row confidently: loss ~1e-3, and the
        # label's gradient entry p_y - 1 is that small too)
        assert abs(host(loss)[0] - l_ref) <= TOL * abs(l_ref), step
        for k in P:
            assert rel_l2(host(G[k]), g_ref[k]) <= TOL, (step, k)
            assert rel_l2(host(P[k]), new_ref[k]) <= TOL, (step, k)
        W = new_ref


def test_fused_mlp_step_limits(ctx):
    d = syn.mlp_inputs(seed=1)
    P = {k: dev(d[k]) for k in ("W1", "b1", "W2", "b2")}
    loss = zeros((1,))
    big = zeros((4096, 3))
    with pytest.raises(tt.TTError, match="64 KB"):
        tt.tt_mlp_step(ctx, big, dev(np.zeros(4096), "i32"), P["W1"], P["b1"], P["W2"], P["b2"],
                       0.1, loss)
    bad = d["labels"].copy()
    bad[5] = 4                          # outside [0, C)
    tt.tt_mlp_step(ctx, dev(d["x"]), dev(bad, "i32"), P["W1"], P["b1"], P["W2"], P["b2"], 0.1, loss)
    with pytest.raises(tt.TTError, match="outside"):
        ctx.sync()
    assert np.isnan(host(loss)[0])
