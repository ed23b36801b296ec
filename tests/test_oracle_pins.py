"""Pins of the CPU oracle against what the pages and the mathematics fix.

Closed forms, printed worked examples, invariants, brute force on tiny inputs
and special cases that reduce to textbook results.  CPU only.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import gpt2 as og
from tests.conftest import rel_l2


# ----------------------------------------------------------- worked examples

def test_scalar_product_worked_example(golden):
    """c = a*b with a=2, b=3: c=6, dc/da=3 (=b), dc/db=2 (=a) — as a 1x1x1 linear."""
    ex = golden("worked_examples.json")["scalar_product"]
    x = np.array([[ex["a"]]])
    W = np.array([[ex["b"]]])
    y = oracle.linear_fwd(x, W)
    dx, dW, _ = oracle.linear_bwd(x, W, np.ones((1, 1)), with_bias=False)
    assert y[0, 0] == ex["c"]
    assert dx[0, 0] == ex["dc_da"]
    assert dW[0, 0] == ex["dc_db"]


def test_gradient_accumulation_two_consumers(golden):
    """x feeds y = 2x and z = 3x: the gradient of x is 2 + 3 = 5."""
    ex = golden("worked_examples.json")["gradient_accumulation"]
    x = np.array([[1.0]])
    W = np.array([[ex["y_coeff"], ex["z_coeff"]]])
    dx, _, _ = oracle.linear_bwd(x, W, np.ones((1, 2)), with_bias=False)
    assert dx[0, 0] == ex["dx"]
    # the same through two separate consumers whose grads are summed
    d1, _, _ = oracle.linear_bwd(x, W[:, :1], np.ones((1, 1)), with_bias=False)
    d2, _, _ = oracle.linear_bwd(x, W[:, 1:], np.ones((1, 1)), with_bias=False)
    assert (d1 + d2)[0, 0] == ex["dx"]


# ------------------------------------------------------------- brute force

def test_linear_matches_triple_loops():
    rng = np.random.default_rng(0)
    M, K, N = 3, 4, 5
    x = rng.standard_normal((M, K))
    W = rng.standard_normal((K, N))
    b = rng.standard_normal(N)
    dy = rng.standard_normal((M, N))
    y = oracle.linear_fwd(x, W, b)
    dx, dW, db = oracle.linear_bwd(x, W, dy)
    for i in range(M):
        for j in range(N):
            s = b[j]
            for k in range(K):
                s += x[i, k] * W[k, j]
            assert abs(y[i, j] - s) < 1e-12
    for i in range(M):
        for k in range(K):
            s = 0.0
            for j in range(N):
                s += dy[i, j] * W[k, j]
            assert abs(dx[i, k] - s) < 1e-12
    for k in range(K):
        for j in range(N):
            s = 0.0
            for i in range(M):
                s += x[i, k] * dy[i, j]
            assert abs(dW[k, j] - s) < 1e-12
    for j in range(N):
        assert abs(db[j] - sum(dy[i, j] for i in range(M))) < 1e-12


def test_attention_matches_scalar_loops():
    """Per-row brute force: scores / sqrt(hs), j <= i only, softmax, weighted sum."""
    rng = np.random.default_rng(1)
    B, T, NH, hs = 1, 4, 2, 3
    C = NH * hs
    qkv = rng.standard_normal((B, T, 3 * C))
    out, lse = oracle.attention_fwd(qkv, NH)
    for h in range(NH):
        for i in range(T):
            q = qkv[0, i, h * hs:(h + 1) * hs]
            sc = []
            for j in range(i + 1):
                k = qkv[0, j, C + h * hs:C + (h + 1) * hs]
                sc.append(sum(q[d] * k[d] for d in range(hs)) / math.sqrt(hs))
            den = sum(math.exp(s) for s in sc)
            assert abs(lse[0, h, i] - math.log(den)) < 1e-12
            for d in range(hs):
                num = sum(math.exp(sc[j]) * qkv[0, j, 2 * C + h * hs + d] for j in range(i + 1))
                assert abs(out[0, i, h * hs + d] - num / den) < 1e-12


def test_cross_entropy_matches_scalar_formula_large_logits():
    """-log(exp(z_y) / sum exp(z)), evaluated by hand with a shifted exponent;
    logits of magnitude 1e3 must not overflow."""
    rng = np.random.default_rng(2)
    N, V = 3, 7
    z = rng.standard_normal((N, V)) * 1000.0
    y = np.array([0, 3, 6])
    loss, dz = oracle.cross_entropy_fwdbwd(z, y)
    tot = 0.0
    for n in range(N):
        m = max(z[n])
        s = sum(math.exp(z[n, v] - m) for v in range(V))
        tot += -(z[n, y[n]] - m - math.log(s))
        for v in range(V):
            p = math.exp(z[n, v] - m) / s
            assert abs(dz[n, v] - (p - (1.0 if v == y[n] else 0.0)) / N) < 1e-15
    assert abs(loss - tot / N) < 1e-9


# ---------------------------------------------------------- closed forms

def test_softmax_rows_sum_to_one_and_dz_rows_sum_to_zero():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((6, 11)) * 5
    p = oracle.softmax_rows(z)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-14)
    _, dz = oracle.cross_entropy_fwdbwd(z, np.arange(6) % 11)
    assert np.allclose(dz.sum(-1), 0.0, atol=1e-15)


def test_ce_uniform_logits_is_log_vocab():
    """All logits equal: loss = ln V exactly; dz = (1/V - onehot)/N."""
    V, N = 50257, 4
    z = np.full((N, V), 0.37)
    y = np.array([0, 17, 50256, 9])
    loss, dz = oracle.cross_entropy_fwdbwd(z, y)
    assert abs(loss - 10.82490511970208) < 1e-12
    exp = np.full((N, V), 1.0 / V)
    exp[np.arange(N), y] -= 1.0
    assert np.allclose(dz, exp / N, atol=1e-18, rtol=1e-12)


def test_ce_four_classes_zero_head_is_log4():
    """Tiny classifier with W2 = 0, b2 = 0: logits all zero, loss = ln 4."""
    rng = np.random.default_rng(4)
    loss, grads, _, z = og.mlp_step(rng.standard_normal((64, 3)), rng.standard_normal((3, 32)),
                                    rng.standard_normal(32), np.zeros((32, 4)), np.zeros(4),
                                    rng.integers(0, 4, 64))
    assert np.all(z == 0)
    assert abs(loss - 1.3862943611198906) < 1e-15


def test_lmhead_zero_weight_closed_form():
    """W_emb = 0: loss = ln V, dHidden = 0, dW[v] = sum_n (1/V - [y_n = v]) h_n / N."""
    rng = np.random.default_rng(5)
    N, C, V = 5, 4, 9
    h = rng.standard_normal((N, C))
    y = np.array([1, 1, 8, 0, 3])
    loss, dh, dwte, _ = oracle.lmhead_ce_fwdbwd(h, np.zeros((V, C)), y)
    assert abs(loss - math.log(V)) < 1e-14
    assert np.all(dh == 0)
    exp = np.zeros((V, C))
    for v in range(V):
        for n in range(N):
            exp[v] += ((1.0 / V) - (1.0 if y[n] == v else 0.0)) * h[n] / N
    assert np.allclose(dwte, exp, atol=1e-15)


def test_attention_special_cases():
    rng = np.random.default_rng(6)
    B, T, NH, hs = 2, 7, 3, 4
    C = NH * hs
    qkv = rng.standard_normal((B, T, 3 * C))
    # V = ones -> every output is 1
    q1 = qkv.copy()
    q1[:, :, 2 * C:] = 1.0
    o, _ = oracle.attention_fwd(q1, NH)
    assert np.allclose(o, 1.0, atol=1e-14)
    # Q = 0 -> scores all 0 -> output i is the mean of v over j <= i
    q2 = qkv.copy()
    q2[:, :, :C] = 0.0
    o, lse = oracle.attention_fwd(q2, NH)
    v = q2[:, :, 2 * C:]
    prefix = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    assert np.allclose(o, prefix, atol=1e-14)
    assert np.allclose(lse, np.log(np.arange(1, T + 1))[None, None, :], atol=1e-14)
    # T = 1 -> output equals v
    o, _ = oracle.attention_fwd(qkv[:, :1], NH)
    assert np.allclose(o, qkv[:, :1, 2 * C:], atol=1e-14)


def test_attention_is_causal():
    """Perturbing positions after i leaves output i (and its gradients' use) unchanged."""
    rng = np.random.default_rng(7)
    B, T, NH = 1, 9, 2
    C = 6
    qkv = rng.standard_normal((B, T, 3 * C))
    o1, _ = oracle.attention_fwd(qkv, NH)
    q2 = qkv.copy()
    q2[:, 5:] += rng.standard_normal((B, T - 5, 3 * C))
    o2, _ = oracle.attention_fwd(q2, NH)
    assert np.array_equal(o1[:, :5], o2[:, :5])
    assert not np.allclose(o1[:, 5:], o2[:, 5:])


def test_layernorm_invariants():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 16)) * 3 + 2
    eps = 1e-5
    y, mean, rstd = oracle.layernorm_fwd(x, np.ones(16), np.zeros(16), eps)
    var = x.var(axis=-1)
    assert np.allclose(y.mean(-1), 0.0, atol=1e-14)
    assert np.allclose(y.var(-1), var / (var + eps), atol=1e-13)
    # shift invariance of the input -> every row of dx sums to zero
    dy = rng.standard_normal((5, 16))
    g = rng.standard_normal(16)
    dx, dg, db = oracle.layernorm_bwd(x, mean, rstd, g, dy)
    assert np.allclose(dx.sum(-1), 0.0, atol=1e-12)
    assert np.allclose(db, dy.sum(0))
    # scale invariance (up to eps): dx is orthogonal to x - mean per row
    assert np.allclose(((x - mean[:, None]) * dx).sum(-1), 0.0, atol=1e-5)


def test_gelu_special_values_and_identities():
    assert oracle.gelu_fwd(np.array(0.0)) == 0.0
    assert abs(oracle.ops.gelu_grad(np.array(0.0)) - 0.5) < 1e-15
    assert abs(oracle.gelu_fwd(np.array(12.0)) - 12.0) < 1e-12
    assert abs(oracle.gelu_fwd(np.array(-12.0))) < 1e-12
    x = np.linspace(-8, 8, 401)
    # 0.5x(1+tanh u) - 0.5(-x)(1+tanh(-u)) = x for an odd u(x)
    assert np.allclose(oracle.gelu_fwd(x) - oracle.gelu_fwd(-x), x, atol=1e-13)
    # the tanh form approximates x * Phi(x) to a few 1e-4
    exact = np.array([0.5 * t * (1 + math.erf(t / math.sqrt(2))) for t in x])
    assert np.max(np.abs(oracle.gelu_fwd(x) - exact)) < 5e-4


def test_gelu_matches_torch_tanh_approximation():
    torch = pytest.importorskip("torch")
    x = np.linspace(-10, 10, 2001)
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    ty = torch.nn.functional.gelu(tx, approximate="tanh")
    ty.sum().backward()
    assert np.allclose(oracle.gelu_fwd(x), ty.detach().numpy(), atol=1e-14)
    assert np.allclose(oracle.ops.gelu_grad(x), tx.grad.numpy(), atol=1e-13)


def test_block_with_zero_weights_is_identity():
    rng = np.random.default_rng(9)
    B, T, C, NH = 2, 5, 8, 2
    w = {k: np.zeros(s) for k, s in [("ln1_g", C), ("ln1_b", C), ("w_qkv", (C, 3 * C)),
                                      ("b_qkv", 3 * C), ("w_proj", (C, C)), ("b_proj", C),
                                      ("ln2_g", C), ("ln2_b", C), ("w_fc", (C, 4 * C)),
                                      ("b_fc", 4 * C), ("w_fcp", (4 * C, C)), ("b_fcp", C)]}
    w["ln1_g"] = np.ones(C)
    w["ln2_g"] = np.ones(C)
    x = rng.standard_normal((B, T, C))
    dy = rng.standard_normal((B, T, C))
    y, cache = og.block_fwd(x, w, NH)
    dx, _ = og.block_bwd(cache, w, dy, NH)
    assert np.array_equal(y, x)
    assert np.array_equal(dx, dy)


def test_parameter_counts(golden):
    g = golden("gpt2_124m_config.json")
    cfg = og.GPTConfig(n_layer=g["num_layers"], n_embd=g["channels"], n_head=g["num_heads"],
                       vocab=g["vocab_size"], block_size=g["max_seq_len"])
    assert og.param_count(cfg, vocab_rows=g["padded_vocab_size"]) == g["num_parameters"]
    assert og.param_count(cfg) == 124439808
    cfg350 = og.GPTConfig(n_layer=24, n_embd=1024, n_head=16)
    assert og.param_count(cfg350) == 354823168


def test_adamw_first_step_closed_form():
    """From m = v = 0 at t = 1: m_hat = g, v_hat = g^2, so
    w1 = w0 - lr * (g / (|g| + eps) + wd * w0)."""
    w = np.array([0.5, -1.0, 2.0])
    g = np.array([0.1, -3.0, 0.0])
    lr, wd, eps = 1e-2, 0.1, 1e-8
    w1, m1, v1 = oracle.adamw_update(w, g, np.zeros(3), np.zeros(3), lr, 0.9, 0.95, eps, wd, 1)
    assert np.allclose(w1, w - lr * (g / (np.abs(g) + eps) + wd * w), atol=1e-16)
    assert np.allclose(m1, 0.1 * g) and np.allclose(v1, 0.05 * g * g)


def test_adamw_matches_torch_over_three_steps():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(10)
    w0 = rng.standard_normal(7)
    gs = [rng.standard_normal(7) for _ in range(3)]
    p = torch.tensor(w0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=3e-4, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)
    w, m, v = w0.copy(), np.zeros(7), np.zeros(7)
    for t, g in enumerate(gs, start=1):
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        w, m, v = oracle.adamw_update(w, g, m, v, 3e-4, 0.9, 0.95, 1e-8, 0.1, t)
    assert np.allclose(w, p.detach().numpy(), atol=1e-15, rtol=1e-13)


def test_sgd_step():
    w = np.array([1.0, -2.0])
    g = np.array([0.5, 0.25])
    assert np.array_equal(oracle.sgd_update(w, g, 0.1), w - 0.1 * g)
    assert np.allclose(oracle.sgd_update(w, g, 0.1), [0.95, -2.025], atol=1e-15)


def test_embedding_fwd_bwd_by_hand():
    wte = np.arange(12.0).reshape(4, 3)
    wpe = np.arange(6.0).reshape(2, 3) * 10
    tok = np.array([[3, 3], [0, 2]])
    x0 = oracle.embed_fwd(tok, wte, wpe)
    assert np.array_equal(x0[0, 1], wte[3] + wpe[1])
    assert np.array_equal(x0[1, 0], wte[0] + wpe[0])
    dx0 = np.ones((2, 2, 3))
    dwte, dwpe = oracle.embed_bwd(tok, dx0, 4, 2)
    assert np.array_equal(dwte[3], [2, 2, 2])      # token 3 used twice
    assert np.array_equal(dwte[1], [0, 0, 0])
    assert np.array_equal(dwpe, np.full((2, 3), 2.0))


def test_initial_loss_near_log_vocab():
    """Random init N(0, 0.02): logits z_v ~ N(0, 0.02^2 * C), so the expected
    loss is about ln V + 0.02^2 * C / 2 (statistical, about +-0.1)."""
    cfg = og.GPTConfig(n_layer=1, n_embd=768, n_head=12, vocab=50257, block_size=64)
    from autograd_transformer_amd import synthetic as syn
    shape = syn.ModelShape(1, 768, 12, 50257, 64)
    p = {k: v.astype(np.float64) for k, v in syn.gpt2_params(shape, seed=11).items()}
    tok, tgt = syn.gpt2_tokens(1, 32, 50257, seed=11)
    loss, _ = og.model_fwd_bwd(p, tok, tgt, cfg)
    assert abs(loss - (math.log(50257) + 0.02 ** 2 * 768 / 2)) < 0.1


# ------------------------------------------------------------- bf16 rule

def test_round_bf16_ties_and_specials():
    rb = oracle.round_bf16
    assert rb(np.array(1.0 + 2 ** -8)) == 1.0                  # tie -> even (down)
    assert rb(np.array(1.0 + 3 * 2 ** -8)) == 1.0 + 2 ** -6    # tie -> even (up)
    assert rb(np.array(1.0 + 2 ** -8 + 2 ** -30)) == 1.0 + 2 ** -7
    assert rb(np.array(-1.0 - 2 ** -8)) == -1.0
    assert np.isnan(rb(np.array(np.nan)))
    assert np.isinf(rb(np.array(3.4e38)))
    assert rb(np.array(3.0)) == 3.0


def test_round_bf16_matches_torch_on_float32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        rng.standard_normal(2000) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_mode_is_close_to_f32_mode():
    """Storage rounding perturbs the step only at the bf16 level."""
    from autograd_transformer_amd import synthetic as syn
    cfg = og.GPTConfig(n_layer=2, n_embd=64, n_head=4, vocab=97, block_size=16)
    shape = syn.ModelShape(2, 64, 4, 97, 16)
    p = {k: v.astype(np.float64) for k, v in syn.gpt2_params(shape, seed=13, bias_std=0.02).items()}
    tok, tgt = syn.gpt2_tokens(2, 16, 97, seed=13)
    l32, g32 = og.model_fwd_bwd(p, tok, tgt, cfg, "f32")
    l16, g16 = og.model_fwd_bwd(p, tok, tgt, cfg, "bf16")
    assert abs(l32 - l16) / l32 < 1e-2
    for k in g32:
        assert rel_l2(g16[k], g32[k]) < 5e-2, k


# ------------------------------------------------------------ greedy decoding

def test_argmax_lowest_index_on_ties_and_first_nan():
    z = np.array([[1.0, 3.0, 3.0, 2.0],
                  [2.0, 2.0, 2.0, 2.0],
                  [-np.inf, -np.inf, -np.inf, -np.inf],
                  [0.0, np.nan, 5.0, np.nan],
                  [-1.0, -0.5, -0.5, -7.0]])
    assert oracle.argmax_rows(z).tolist() == [1, 0, 0, 1, 1]


def _tiny_cfg():
    return og.GPTConfig(n_layer=2, n_embd=8, n_head=2, vocab=13, block_size=8)


def _tiny_params(cfg, seed=7):
    rng = np.random.default_rng(seed)
    p = {}
    for name, shape in og.param_shapes(cfg):
        std = 0.3 if name.split(".")[-1] in ("ln1_g", "ln2_g") or name == "lnf_g" else 0.5
        base = 1.0 if name.endswith("_g") else 0.0
        p[name] = base + std * rng.standard_normal(shape)
    return p


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_logits_of_a_prefix_do_not_depend_on_later_tokens(mode):
    """Causality: the logits of position t from the prefix 0..t equal the
    logits of position t in the forward over the whole sequence, which is what
    lets a decoder reuse cached keys and values."""
    cfg = _tiny_cfg()
    p = _tiny_params(cfg)
    tok = np.random.default_rng(3).integers(0, cfg.vocab, size=(2, 7))
    full = og.model_logits(p, tok, cfg, mode)
    for t in range(7):
        pre = og.model_logits(p, tok[:, :t + 1], cfg, mode)
        assert np.allclose(pre[:, t], full[:, t], rtol=1e-12, atol=1e-12), t
    # and a later token does change a later position
    tok2 = tok.copy()
    tok2[:, 3] = (tok2[:, 3] + 1) % cfg.vocab
    assert not np.allclose(og.model_logits(p, tok2, cfg, mode)[:, 5], full[:, 5])


def test_greedy_copy_model_closed_form():
    """Every block zero, token table 4 * one-hot rows, no position table: the
    residual stream is wte[tok], so the logits are closed form and the argmax
    is the current token -- greedy decoding repeats the prompt's last token."""
    C, V = 16, 13
    cfg = og.GPTConfig(n_layer=2, n_embd=C, n_head=2, vocab=V, block_size=8)
    p = {name: np.zeros(shape) for name, shape in og.param_shapes(cfg)}
    for name in p:
        if name.endswith("_g"):
            p[name][:] = 1.0
    p["wte"][:V, :V] = 4.0 * np.eye(V)
    prompt = np.array([[3, 9, 7], [0, 12, 5]])
    seq, steps = og.greedy_generate(p, prompt, 4, cfg, "f32")
    assert seq[:, 3:].tolist() == [[7] * 4, [5] * 4]
    sd = math.sqrt(16.0 / C * (1.0 - 1.0 / C) + 1e-5)
    for b, v in enumerate([7, 5]):
        want = 4.0 * (4.0 * (np.arange(V) == v) - 4.0 / C) / sd
        assert np.allclose(steps[0, b], want, rtol=1e-12, atol=1e-12)


def test_greedy_tokens_are_argmaxes_of_the_full_forward():
    cfg = _tiny_cfg()
    p = _tiny_params(cfg, seed=11)
    prompt = np.random.default_rng(5).integers(0, cfg.vocab, size=(3, 2))
    seq, steps = og.greedy_generate(p, prompt, 5, cfg, "f32")
    z = og.model_logits(p, seq, cfg, "f32")
    for j in range(5):
        assert np.array_equal(seq[:, 2 + j], np.argmax(z[:, 1 + j], axis=-1))
        assert np.allclose(steps[j], z[:, 1 + j], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ gradient clipping

def test_clip_grad_norm_three_four_five():
    """Norm of (3, 4) is 5: above max_norm the gradients scale by
    max_norm / (5 + 1e-6), below it they are unchanged."""
    g = {"a": np.array([3.0]), "b": np.array([[4.0, 0.0]])}
    out, n = oracle.clip_grad_norm(g, 1.0)
    assert n == 5.0
    c = 1.0 / (5.0 + 1e-6)
    assert out["a"].tolist() == [3.0 * c] and out["b"].tolist() == [[4.0 * c, 0.0]]
    out, n = oracle.clip_grad_norm(g, 10.0)
    assert n == 5.0 and out["a"].tolist() == [3.0] and out["b"].tolist() == [[4.0, 0.0]]


def test_clip_grad_norm_brute_force_and_torch():
    rng = np.random.default_rng(12)
    g = {f"t{i}": rng.standard_normal(rng.integers(1, 40, size=2)) for i in range(6)}
    out, n = oracle.clip_grad_norm(g, 0.5)
    s = 0.0
    for v in g.values():
        for x in v.reshape(-1):
            s += float(x) * float(x)
    assert abs(n - math.sqrt(s)) <= 1e-12 * n
    import torch
    ts = [torch.tensor(v, dtype=torch.float64, requires_grad=True) for v in g.values()]
    for t, v in zip(ts, g.values()):
        t.grad = torch.tensor(v, dtype=torch.float64)
    tn = torch.nn.utils.clip_grad_norm_(ts, 0.5)
    assert abs(float(tn) - n) <= 1e-12 * n
    for t, k in zip(ts, g):
        assert np.allclose(t.grad.numpy(), out[k], rtol=1e-12, atol=0)


# ------------------------------------------------ fp16 and loss scaling

def test_round_fp16_ties_range_and_subnormals():
    """binary16 by hand: 11 significant bits, ties to even, largest finite
    65504 (65520 is the midpoint to 2**16 and rounds up to infinity),
    subnormal step 2**-24 -- and one rounding of the float64 value (a detour
    through float32 would turn 1 + 2**-11 + 2**-30 into the tie 1 + 2**-11
    and then into 1)."""
    x = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -30,
                  65504.0, 65519.99, 65520.0, -70000.0, 2.0 ** -25, 3 * 2.0 ** -26,
                  2.0 ** -25 + 2.0 ** -40, 2.0 ** -14, -0.0, 0.1])
    want = np.array([1.0, 1 + 2.0 ** -9, 1 + 2.0 ** -10, 65504.0, 65504.0, np.inf, -np.inf,
                     0.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -14, -0.0,
                     1638 * 2.0 ** -14])   # 0.1 = 1.6 * 2**-4; 1.6 * 1024 = 1638.4 -> 1638
    got = oracle.round_fp16(x)
    assert np.array_equal(got, want)
    assert np.signbit(got[11])
    assert np.isnan(oracle.round_fp16(np.nan))


def test_loss_scale_update_by_hand():
    """Halve on overflow and restart the count; grow by 1.001 after 1000
    consecutive clean steps."""
    s, g = 65536.0, 0
    s, g = oracle.loss_scale_update(s, g, True)
    assert (s, g) == (32768.0, 0)
    for _ in range(999):
        s, g = oracle.loss_scale_update(s, g, False)
    assert (s, g) == (32768.0, 999)
    s, g = oracle.loss_scale_update(s, g, False)
    assert s == 32768.0 * 1.001 and g == 0
    s, g = oracle.loss_scale_update(s, g, False)
    assert g == 1
    s, g = oracle.loss_scale_update(s, 500, True)
    assert s == 32768.0 * 1.001 / 2 and g == 0


def _fp16_model():
    from autograd_transformer_amd import synthetic as syn
    cfg = og.GPTConfig(n_layer=2, n_embd=64, n_head=4, vocab=97, block_size=16)
    shape = syn.ModelShape(2, 64, 4, 97, 16)
    p = {k: v.astype(np.float64) for k, v in syn.gpt2_params(shape, seed=14, bias_std=0.02).items()}
    tok, tgt = syn.gpt2_tokens(2, 16, 97, seed=14)
    return cfg, p, tok, tgt


def test_power_of_two_loss_scale_is_exact_without_storage_rounding():
    """Scaling the loss gradient by 2**k and dividing the weight gradients by
    it again changes no bit when nothing is rounded to a storage format."""
    cfg, p, tok, tgt = _fp16_model()
    l1, g1 = og.model_fwd_bwd(p, tok, tgt, cfg, "f32")
    l2, g2 = og.model_fwd_bwd(p, tok, tgt, cfg, "f32", loss_scale=2.0 ** 10)
    assert l1 == l2
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k


def test_fp16_mode_rounds_to_fp16():
    """fp16 storage (11 significant bits) stays closer to the unrounded step
    than bf16 storage (8 bits), and is not the unrounded step itself."""
    cfg, p, tok, tgt = _fp16_model()
    _, g32 = og.model_fwd_bwd(p, tok, tgt, cfg, "f32")
    _, gh = og.model_fwd_bwd(p, tok, tgt, cfg, "fp16", loss_scale=1024.0)
    _, gb = og.model_fwd_bwd(p, tok, tgt, cfg, "bf16")
    eh = np.mean([rel_l2(gh[k], g32[k]) for k in g32])
    eb = np.mean([rel_l2(gb[k], g32[k]) for k in g32])
    assert 0 < eh < eb / 3, (eh, eb)
    for k in g32:
        assert rel_l2(gh[k], g32[k]) < 1e-2, k


def test_fp16_step_overflow_is_skipped_and_scale_halves():
    cfg, p, tok, tgt = _fp16_model()
    zeros = {k: np.zeros_like(v) for k, v in p.items()}
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1)
    # 2**40 / N puts the label's dlogit far past 65504: infinity in fp16
    out = og.train_step_scaled(p, zeros, dict(zeros), 1, tok, tgt, cfg, 2.0 ** 40, 7, **hp)
    _, _, new_p, _, _, s, g, skipped = out
    assert skipped and s == 2.0 ** 39 and g == 0
    assert all(new_p[k] is p[k] for k in p)
    # a representable scale: a normal AdamW step on the unscaled gradients
    out = og.train_step_scaled(p, zeros, dict(zeros), 1, tok, tgt, cfg, 1024.0, 7, **hp)
    loss, grads, new_p, new_m, _, s, g, skipped = out
    assert not skipped and s == 1024.0 and g == 8
    _, g_ref = og.model_fwd_bwd(p, tok, tgt, cfg, "fp16", loss_scale=1024.0)
    for k in p:
        w_ref, m_ref, _ = oracle.adamw_update(p[k], g_ref[k], 0, 0, t=1, **hp)
        assert np.array_equal(new_p[k], w_ref) and np.array_equal(new_m[k], m_ref), k
