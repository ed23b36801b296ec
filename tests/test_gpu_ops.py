"""Op-level parity: every libtt op against the float64 oracle on seeded inputs.

Sizes span several GEMM / attention tiles and ragged tails.  Bars: rel-L2 <=
1e-5 in fp32 mode, <= 2e-2 in bf16 mode and <= 1e-2 in fp16 mode; exact for
gathers and for the printed worked examples.  fp16 products need operand rows
that are multiples of 8 elements: other shapes must be refused.
"""

import math

import numpy as np
import pytest

import oracle
import autograd_transformer_amd as tt
from autograd_transformer_amd import synthetic as syn
from tests.conftest import rel_l2
from tests.gpu_util import dev, host, empty, zeros, lowp, store, tol, sync, exact_in

pytestmark = pytest.mark.gpu

MODES = ["f32", "bf16", "fp16"]
MODES_ANY_SHAPE = ["f32", "bf16"]   # products of any row length


@pytest.fixture(scope="module")
def ctx():
    c = tt.Context(arena_bytes=4 << 30)
    yield c
    c.close()


def _inputs(mode, shape, seed, std=1.0):
    return exact_in(mode, syn.normal(seed, shape, std))


def _fp16_refused(ctx, mode, K, N, call):
    """fp16 products with rows that are not multiples of 8 must be refused."""
    if mode != "fp16" or (K % 8 == 0 and N % 8 == 0):
        return False
    with pytest.raises(tt.TTError, match="fp16"):
        call()
    return True


# ------------------------------------------------------------ worked examples

@pytest.mark.parametrize("mode", MODES_ANY_SHAPE)
def test_scalar_product_worked_example(ctx, mode, golden):
    """c = a*b with a=2, b=3 as a 1x1x1 linear: y=6, dy/dx=3, dy/dW=2, exactly."""
    ex = golden("worked_examples.json")["scalar_product"]
    X = dev(np.array([[ex["a"]]]), lowp(mode))
    W = dev(np.array([[ex["b"]]]), lowp(mode))
    Y = empty((1, 1), lowp(mode))
    tt.tt_linear_fwd(ctx, mode, 1, 1, 1, X, W, None, Y)
    dY = dev(np.ones((1, 1)), lowp(mode))
    dX, dW = empty((1, 1)), zeros((1, 1))
    tt.tt_linear_bwd(ctx, mode, 1, 1, 1, X, W, dY, dX, dW)
    sync()
    assert host(Y)[0, 0] == ex["c"]
    assert host(dX)[0, 0] == ex["dc_da"]
    assert host(dW)[0, 0] == ex["dc_db"]


@pytest.mark.parametrize("mode", MODES_ANY_SHAPE)
def test_gradient_accumulation_2_plus_3(ctx, mode, golden):
    ex = golden("worked_examples.json")["gradient_accumulation"]
    X = dev(np.array([[1.0]]), lowp(mode))
    W = dev(np.array([[ex["y_coeff"], ex["z_coeff"]]]), lowp(mode))
    dY = dev(np.ones((1, 2)), lowp(mode))
    dX = empty((1, 1))
    tt.tt_linear_bwd(ctx, mode, 1, 1, 2, X, W, dY, dX)
    sync()
    assert host(dX)[0, 0] == ex["dx"]
    # two consumers, gradients accumulated into one buffer
    W1 = dev(np.array([[ex["y_coeff"]]]), lowp(mode))
    W2 = dev(np.array([[ex["z_coeff"]]]), lowp(mode))
    d1 = dev(np.ones((1, 1)), lowp(mode))
    acc = zeros((1, 1))
    tt.tt_linear_bwd(ctx, mode, 1, 1, 1, X, W1, d1, acc, accumulate_dX=True)
    tt.tt_linear_bwd(ctx, mode, 1, 1, 1, X, W2, d1, acc, accumulate_dX=True)
    sync()
    assert host(acc)[0, 0] == ex["dx"]


# ------------------------------------------------------------------ linear

# (17, 96, 48) and (40, 64, 64): weight gradients whose token reduction is one
# and two 32-deep stages, shorter than the operand ring
SHAPES = [(64, 3, 32), (300, 200, 130), (256, 256, 384), (129, 64, 17), (1000, 768, 2304),
          (4160, 768, 768), (17, 96, 48), (40, 64, 64)]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("epi", ["none", "gelu", "resid"])
def test_linear_fwd(ctx, mode, shape, epi):
    M, K, N = shape
    S = store(mode)
    x = _inputs(mode, (M, K), 100)
    W = _inputs(mode, (K, N), 101, 0.1)
    b = syn.normal(102, (N,), 0.1)
    r = syn.normal(103, (M, N))
    y_ref = oracle.linear_fwd(x, W, b)
    X, Wd, bd = dev(x, lowp(mode)), dev(W, lowp(mode)), dev(b)
    if _fp16_refused(ctx, mode, K, N, lambda: tt.tt_linear_fwd(ctx, mode, M, K, N, X, Wd, bd,
                                                               empty((M, N), "fp16"))):
        return
    if epi == "none":
        Y = empty((M, N), lowp(mode))
        tt.tt_linear_fwd(ctx, mode, M, K, N, X, Wd, bd, Y)
        sync()
        assert rel_l2(host(Y), S(y_ref)) <= tol(mode)
    elif epi == "gelu":
        Y, P = empty((M, N), lowp(mode)), empty((M, N), lowp(mode))
        tt.tt_linear_fwd(ctx, mode, M, K, N, X, Wd, bd, Y, tt.TT_EPI_GELU, None, P)
        sync()
        assert rel_l2(host(P), S(y_ref)) <= tol(mode)
        assert rel_l2(host(Y), S(oracle.gelu_fwd(y_ref))) <= tol(mode)
    else:
        Y = empty((M, N))
        tt.tt_linear_fwd(ctx, mode, M, K, N, X, Wd, bd, Y, tt.TT_EPI_RESIDUAL, dev(r))
        sync()
        assert rel_l2(host(Y), r + y_ref) <= tol(mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", SHAPES)
def test_linear_bwd(ctx, mode, shape):
    M, K, N = shape
    x = _inputs(mode, (M, K), 110)
    W = _inputs(mode, (K, N), 111, 0.1)
    dy = _inputs(mode, (M, N), 112)
    dx_ref, dW_ref, db_ref = oracle.linear_bwd(x, W, dy)
    X, Wd, dY = dev(x, lowp(mode)), dev(W, lowp(mode)), dev(dy, lowp(mode))
    dX = empty((M, K))
    dW0 = syn.normal(113, (K, N))     # += semantics: start from a nonzero buffer
    db0 = syn.normal(114, (N,))
    dW, db = dev(dW0), dev(db0)
    if _fp16_refused(ctx, mode, K, N, lambda: tt.tt_linear_bwd(ctx, mode, M, K, N, X, Wd, dY, dX,
                                                               dW, db)):
        return
    tt.tt_linear_bwd(ctx, mode, M, K, N, X, Wd, dY, dX, dW, db)
    sync()
    assert rel_l2(host(dX), dx_ref) <= tol(mode)
    assert rel_l2(host(dW), dW0 + dW_ref) <= tol(mode)
    assert rel_l2(host(db), db0 + db_ref) <= tol(mode)


@pytest.mark.parametrize("mode", MODES)
def test_linear_bwd_last_element(ctx, mode):
    """The last token's gradient in the last of an odd number of columns: the
    only nonzero of dY.  dW's last column is then exactly that token's input
    row, db's last entry 1 -- an operand range that ended inside its last
    dword once read that element as 0."""
    M, K, N = 33, 16, 17
    x = _inputs(mode, (M, K), 120)
    W = _inputs(mode, (K, N), 121, 0.1)
    dy = np.zeros((M, N))
    dy[M - 1, N - 1] = 1.0
    X, Wd, dY = dev(x, lowp(mode)), dev(W, lowp(mode)), dev(dy, lowp(mode))
    dX, dW, db = empty((M, K)), zeros((K, N)), zeros((N,))
    if _fp16_refused(ctx, mode, K, N, lambda: tt.tt_linear_bwd(ctx, mode, M, K, N, X, Wd, dY, dX,
                                                               dW, db)):
        return
    tt.tt_linear_bwd(ctx, mode, M, K, N, X, Wd, dY, dX, dW, db)
    sync()
    got = host(dW)
    assert np.array_equal(got[:, N - 1], x[M - 1])
    assert not np.any(got[:, : N - 1])
    assert host(db)[N - 1] == 1.0 and not np.any(host(db)[: N - 1])


# --------------------------------------------------------------- layernorm

@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("NC", [(1, 4), (37, 768), (1000, 1024), (5, 4096), (300, 36),
                                (4099, 768), (8195, 100)])
def test_layernorm(ctx, mode, NC):
    N, C = NC
    x = syn.normal(120, (N, C), 2.0) + 0.5
    g = 1.0 + syn.normal(121, (C,), 0.3)
    b = syn.normal(122, (C,), 0.3)
    dy = syn.normal(123, (N, C))
    y_ref, mu_ref, rs_ref = oracle.layernorm_fwd(x, g, b)
    dx_ref, dg_ref, db_ref = oracle.layernorm_bwd(x, mu_ref, rs_ref, g, dy)
    xd, gd, bd = dev(x), dev(g), dev(b)
    y, mu, rs = empty((N, C), lowp(mode)), empty((N,)), empty((N,))
    tt.tt_layernorm_fwd(ctx, mode, N, C, 1e-5, xd, gd, bd, y, mu, rs)
    dx0 = syn.normal(124, (N, C))
    dx, dg, db = dev(dx0), zeros((C,)), zeros((C,))
    tt.tt_layernorm_bwd(ctx, mode, N, C, xd, mu, rs, gd, dev(dy), dx, dg, db)
    sync()
    assert rel_l2(host(y), store(mode)(y_ref)) <= tol(mode)
    assert rel_l2(host(mu), mu_ref) <= 1e-6
    assert rel_l2(host(rs), rs_ref) <= 1e-6
    assert rel_l2(host(dx), dx0 + dx_ref) <= 1e-5
    assert rel_l2(host(dg), dg_ref) <= 1e-5
    assert rel_l2(host(db), db_ref) <= 1e-5


@pytest.mark.parametrize("mode", MODES)
def test_gelu(ctx, mode):
    n = 100003
    x = _inputs(mode, (n,), 130, 3.0)
    dy = _inputs(mode, (n,), 131)
    X, dY = dev(x, lowp(mode)), dev(dy, lowp(mode))
    Y, dX = empty((n,), lowp(mode)), empty((n,), lowp(mode))
    tt.tt_gelu_fwd(ctx, mode, n, X, Y)
    tt.tt_gelu_bwd(ctx, mode, n, X, dY, dX)
    sync()
    S = store(mode)
    assert rel_l2(host(Y), S(oracle.gelu_fwd(x))) <= tol(mode)
    assert rel_l2(host(dX), S(oracle.gelu_bwd(x, dy))) <= tol(mode)
    assert host(Y)[np.argmin(np.abs(x))] == pytest.approx(0.0, abs=1e-3)


def test_gelu_saturation_and_sign(ctx):
    """GELU and its derivative from the far negative tail (exp overflow: the
    sigmoid factor must become exactly 0, not NaN) through zero to the far
    positive tail (GELU(x) = x, derivative 1), element by element in fp32."""
    x = np.array([-1e4, -100, -20, -10, -5, -3, -1, -0.1, -1e-3, 0.0,
                  1e-3, 0.1, 1, 3, 5, 10, 20, 100, 1e4], np.float32)
    n = x.size
    dy = np.ones(n, np.float32)
    X, dY = dev(x), dev(dy)
    Y, dX = empty((n,)), empty((n,))
    tt.tt_gelu_fwd(ctx, "f32", n, X, Y)
    tt.tt_gelu_bwd(ctx, "f32", n, X, dY, dX)
    sync()
    y, g = host(Y), host(dX)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(g))
    y_ref, g_ref = oracle.gelu_fwd(x), oracle.gelu_bwd(x, dy)
    np.testing.assert_allclose(y, y_ref, rtol=4e-6, atol=1e-30)
    np.testing.assert_allclose(g, g_ref, rtol=4e-6, atol=2e-6)
    assert y[x <= -20].max() <= 0.0 and y[x >= 20].tolist() == x[x >= 20].tolist()


# ---------------------------------------------------------------- attention

ATTN = [(2, 1, 2), (1, 77, 3), (2, 256, 2), (1, 300, 1), (1, 1024, 1)]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", ATTN)
def test_attention(ctx, mode, shape):
    B, T, NH = shape
    C = NH * 64
    qkv = _inputs(mode, (B, T, 3 * C), 140)
    dout = _inputs(mode, (B, T, C), 141)
    o_ref, lse_ref = oracle.attention_fwd(qkv, NH)
    S = store(mode)
    o_st = S(o_ref)
    # the backward is checked against the oracle's exact gradient of the
    # stored output's upstream gradient
    dqkv_ref = oracle.attention_bwd(qkv, dout, NH)
    Q = dev(qkv, lowp(mode))
    O, L = empty((B, T, C), lowp(mode)), empty((B, NH, T))
    tt.tt_attn_fwd(ctx, mode, B, T, NH, 64, Q, O, L)
    dQ = empty((B, T, 3 * C), lowp(mode))
    tt.tt_attn_bwd(ctx, mode, B, T, NH, 64, Q, O, L, dev(dout, lowp(mode)), dQ)
    sync()
    assert rel_l2(host(O), o_st) <= tol(mode)
    assert rel_l2(host(L), lse_ref) <= 1e-5
    assert rel_l2(host(dQ), S(dqkv_ref)) <= tol(mode)


# ----------------------------------------------------------- cross-entropy

@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("NV", [(37, 1000), (8, 50257), (300, 13)])
def test_cross_entropy(ctx, mode, NV):
    N, V = NV
    ld = (V + 63) // 64 * 64
    z = _inputs(mode, (N, V), 150, 3.0)
    y = np.random.default_rng(151).integers(0, V, N)
    loss_ref, dz_ref = oracle.cross_entropy_fwdbwd(z, y)
    zp = np.zeros((N, ld))
    zp[:, :V] = z
    Z = dev(zp, lowp(mode))
    loss = empty((1,))
    tt.tt_ce_fwdbwd(ctx, mode, N, V, ld, Z, dev(y, "i32"), loss)
    sync()
    out = host(Z)
    assert abs(host(loss)[0] - loss_ref) / loss_ref <= tol(mode)
    assert rel_l2(out[:, :V], store(mode)(dz_ref)) <= tol(mode)
    assert np.all(out[:, V:] == 0)


@pytest.mark.parametrize("mode", MODES)
def test_cross_entropy_uniform_is_log_v(ctx, mode):
    N, V = 4, 50257
    ld = 50304
    Z = dev(np.full((N, ld), 0.25), lowp(mode))
    loss = empty((1,))
    tt.tt_ce_fwdbwd(ctx, mode, N, V, ld, Z, dev(np.array([0, 5, 50256, 77]), "i32"), loss)
    sync()
    assert host(loss)[0] == pytest.approx(math.log(V), rel=1e-6)
    # closed form dz = (1/V - onehot)/N, as stored in the mode's dtype
    exp = np.full((N, V), 1.0 / V)
    exp[np.arange(N), [0, 5, 50256, 77]] -= 1.0
    exp = store(mode)(exp / N)
    assert np.allclose(host(Z)[:, :V], exp, rtol=1e-5 if mode == "f32" else 8e-3, atol=0)
    if mode == "f32":
        assert np.allclose(host(Z)[:, :V].sum(-1), 0.0, atol=1e-6)


# ----------------------------------------------------------- embeddings

def test_embedding_fwd_exact_and_bwd(ctx):
    B, T, C, V = 3, 50, 768, 1000
    wte = syn.normal(160, (V, C), 0.02)
    wpe = syn.normal(161, (T + 7, C), 0.02)
    tok = np.random.default_rng(162).integers(0, V, (B, T))
    tok[0, :5] = 7                      # repeated ids accumulate
    x0 = empty((B, T, C))
    tt.tt_embed_fwd(ctx, B, T, C, V, dev(tok, "i32"), dev(wte), dev(wpe), x0)
    dx0 = syn.normal(163, (B, T, C))
    dwte, dwpe = zeros((V, C)), zeros((T + 7, C))
    tt.tt_embed_bwd(ctx, B, T, C, V, dev(tok, "i32"), dev(dx0), dwte, dwpe)
    sync()
    ref = oracle.embed_fwd(tok, wte, wpe).astype(np.float32)   # one fp32 rounding of the sum
    assert np.array_equal(host(x0).astype(np.float32), ref)
    dwte_ref, dwpe_ref = oracle.embed_bwd(tok, dx0, V, T + 7)
    assert rel_l2(host(dwte), dwte_ref) <= 1e-6
    assert rel_l2(host(dwpe), dwpe_ref) <= 1e-6


def test_embedding_out_of_range_is_reported(ctx):
    B, T, C, V = 1, 4, 64, 10
    x0 = empty((B, T, C))
    tok = dev(np.array([[1, 2, 10, 3]]), "i32")
    tt.tt_embed_fwd(ctx, B, T, C, V, tok, dev(np.zeros((V, C))), dev(np.zeros((T, C))), x0)
    with pytest.raises(tt.TTError) as e:
        ctx.sync()
    assert e.value.status == -7
    assert np.isnan(host(x0)[0, 2]).all() and not np.isnan(host(x0)[0, 1]).any()
    ctx.sync()  # the flag was cleared


# ----------------------------------------------------------- optimisers

def test_adamw_matches_oracle(ctx):
    n = 10001
    w0, g = syn.normal(170, (n,)), syn.normal(171, (n,))
    m0, v0 = syn.normal(172, (n,), 0.1), np.abs(syn.normal(173, (n,), 0.1))
    W, G, Mm, Vv = dev(w0), dev(g), dev(m0), dev(v0)
    Wl = empty((n,), "bf16")
    tt.tt_adamw_step(ctx, [dict(w=W, g=G, m=Mm, v=Vv, w_lowp=Wl)], 3e-4, 0.9, 0.95, 1e-8, 0.1, 3)
    sync()
    w_ref, m_ref, v_ref = oracle.adamw_update(w0, g, m0, v0, 3e-4, 0.9, 0.95, 1e-8, 0.1, 3)
    # The new weight is stored in float32: each element within 2 float32 ulps
    # of the larger of old and new weight, plus 1e-5 of the update (the
    # update is computed in float32 too; a ~3e-4 update on |w| ~ 1 carries
    # ~4e-4 relative rounding of its own, so it is not compared on its own).
    ulp = np.spacing(np.maximum(np.abs(w_ref), np.abs(w0)).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(host(W) - w_ref) <= 2 * ulp + 1e-5 * np.abs(w_ref - w0))
    assert rel_l2(host(W), w_ref) <= 1e-7
    assert rel_l2(host(Mm), m_ref) <= 1e-6 and rel_l2(host(Vv), v_ref) <= 1e-6
    assert np.array_equal(host(Wl), oracle.round_bf16(host(W)))


def test_adamw_first_step_closed_form(ctx):
    w0 = np.array([0.5, -1.0, 2.0, 0.25])
    g = np.array([0.1, -3.0, 0.0, 1e-3])
    W, G, Mm, Vv = dev(w0), dev(g), zeros((4,)), zeros((4,))
    tt.tt_adamw_step(ctx, [dict(w=W, g=G, m=Mm, v=Vv)], 1e-2, 0.9, 0.95, 1e-8, 0.1, 1)
    sync()
    exp = w0 - 1e-2 * (g / (np.abs(g) + 1e-8) + 0.1 * w0)
    assert np.allclose(host(W), exp, rtol=1e-6, atol=1e-7)


def test_sgd(ctx):
    w0, g = syn.normal(180, (777,)), syn.normal(181, (777,))
    W = dev(w0)
    tt.tt_sgd_step(ctx, W, dev(g), 0.1)
    sync()
    assert np.array_equal(host(W).astype(np.float32), (w0 - np.float32(0.1) * g).astype(np.float32)) or \
        rel_l2(host(W), oracle.sgd_update(w0, g, 0.1)) <= 1e-7


# --------------------------------------------------------- LM head + CE

@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("NCV", [(300, 64, 1000), (256, 768, 5000)])
def test_lmhead_ce(ctx, mode, NCV):
    N, C, V = NCV
    d = syn.lmhead_inputs(seed=190, N=N, C=C, V=V)
    h, w, y = d["h"], d["wte"], d["targets"]
    S = store(mode)
    loss_ref, dh_ref, dw_ref, _ = oracle.lmhead_ce_fwdbwd(h, w, y, S, S)
    loss, dh = empty((1,)), empty((N, C))
    dw0 = syn.normal(191, (V, C), 1e-3)
    dw = dev(dw0)
    tt.tt_lmhead_ce_fwdbwd(ctx, mode, N, C, V, dev(h, lowp(mode)), dev(w, lowp(mode)),
                           dev(y, "i32"), loss, dh, dw)
    sync()
    assert abs(host(loss)[0] - loss_ref) / loss_ref <= tol(mode)
    assert rel_l2(host(dh), dh_ref) <= tol(mode)
    assert rel_l2(host(dw) - dw0, dw_ref) <= tol(mode)


def test_lmhead_ce_full_size_against_oracle_samples(ctx):
    """hidden [8192, 768] x W_emb [50257, 768] in bf16: loss, the norms of
    dHidden and dW_emb and 256 sampled entries of each against the values the
    oracle wrote (tests/golden/make_lmhead_ce_full.py)."""
    import json
    import os
    from tests.conftest import GOLDEN
    with open(os.path.join(GOLDEN, "lmhead_ce_n8192_c768_v50257_bf16.json")) as f:
        ref = json.load(f)
    w = ref["workload"]
    N, C, V = w["N"], w["C"], w["V"]
    d = syn.lmhead_inputs(seed=w["seed"], N=N, C=C, V=V)
    loss, dh, dw = empty((1,)), empty((N, C)), zeros((V, C))
    tt.tt_lmhead_ce_fwdbwd(ctx, "bf16", N, C, V, dev(d["h"], "bf16"), dev(d["wte"], "bf16"),
                           dev(d["targets"], "i32"), loss, dh, dw)
    sync()
    assert abs(host(loss)[0] - ref["loss"]) / ref["loss"] <= 2e-2
    for name, got in (("dh", host(dh)), ("dwte", host(dw))):
        r = ref["tensors"][name]
        flat = got.reshape(-1)
        assert abs(np.linalg.norm(flat) - r["norm"]) / r["norm"] <= 2e-2, name
        assert rel_l2(flat[np.array(r["idx"])], np.array(r["val"])) <= 2e-2, name


def test_lmhead_ce_full_size_elementwise(ctx):
    """The LM head + CE workload at its benchmarked size (hidden [8192, 768] x
    W_emb [50257, 768], bf16) element by element against the oracle run here:
    the loss, the whole of dHidden and dW_emb (rel-L2), their last rows (the
    ragged end of the token and vocabulary ranges) and the dW_emb rows of the
    targets."""
    N, C, V = 8192, 768, 50257
    d = syn.lmhead_inputs(seed=4, N=N, C=C, V=V)
    loss, dh, dw = empty((1,)), empty((N, C)), zeros((V, C))
    tt.tt_lmhead_ce_fwdbwd(ctx, "bf16", N, C, V, dev(d["h"], "bf16"), dev(d["wte"], "bf16"),
                           dev(d["targets"], "i32"), loss, dh, dw)
    sync()
    l_ref, dh_ref, dw_ref, _ = oracle.lmhead_ce_fwdbwd(
        d["h"].astype(np.float64), d["wte"].astype(np.float64), d["targets"],
        store_logits=oracle.round_bf16, store_dlogits=oracle.round_bf16)
    got_dh, got_dw = host(dh), host(dw)
    errs = {"loss": abs(host(loss)[0] - l_ref) / l_ref,
            "dh": rel_l2(got_dh, dh_ref), "dwte": rel_l2(got_dw, dw_ref),
            "dh last row": rel_l2(got_dh[-1], dh_ref[-1]),
            "dwte last rows": rel_l2(got_dw[V - 81:], dw_ref[V - 81:]),
            "dwte target rows": rel_l2(got_dw[d["targets"][-64:]], dw_ref[d["targets"][-64:]])}
    print({k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: e for k, e in errs.items() if not e <= 2e-2}
    assert not bad, bad


# ------------------------------------------------------------ error paths

def test_errors_are_reported_not_raised_by_kernels(ctx):
    with pytest.raises(tt.TTError) as e:
        tt.tt_linear_fwd(ctx, "f32", 0, 3, 3, empty((1, 3)), empty((3, 3)), None, empty((1, 3)))
    assert e.value.status == -1
    with pytest.raises(tt.TTError) as e:
        tt.tt_attn_fwd(ctx, "f32", 1, 8, 2, 32, empty((1, 8, 192)), empty((1, 8, 64)), empty((1, 2, 8)))
    assert e.value.status == -6
    with pytest.raises(tt.TTError) as e:
        tt.tt_layernorm_fwd(ctx, "f32", 4, 6, 1e-5, empty((4, 6)), empty((6,)), empty((6,)), empty((4, 6)))
    assert e.value.status == -1


def test_arena_exhaustion_and_reset(ctx):
    used0, cap = ctx.usage()
    with pytest.raises(tt.TTError) as e:
        ctx.alloc(cap + 1)
    assert e.value.status == -2
    ctx.mark()
    a = ctx.alloc(1000)
    b = ctx.alloc(10)
    assert a % 256 == 0 and b % 256 == 0 and b >= a + 1000
    ctx.reset()
    assert ctx.alloc(1000) == a
    ctx.reset()


def test_stale_and_null_handles():
    import ctypes
    L = tt.lib()
    L.tt_ctx_destroy(None)          # NULL-safe
    L.tt_model_destroy(None)
    fake = ctypes.create_string_buffer(256)   # zeroed: magic word does not match
    assert L.tt_ctx_sync(ctypes.cast(fake, ctypes.c_void_p)) == -4
    assert L.tt_ctx_sync(None) == -1
