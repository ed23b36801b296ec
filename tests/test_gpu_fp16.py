"""fp16 training with dynamic loss scaling against the oracle.

* a small model's step in TT_FP16 at a fixed scale: loss, every (unscaled)
  gradient and the post-AdamW weights against oracle.model_fwd_bwd(mode="fp16",
  loss_scale=...) and oracle.adamw_update (bar: rel-L2 <= 1e-2);
* an overflowing scale: the step is dropped (weights and moments unchanged
  bit for bit), the flag is raised, the scale halves -- then a sane scale
  trains again (oracle.train_step_scaled decides every case);
* the scale schedule over several steps against oracle.loss_scale_update;
* the GPT-2 124M step in fp16 at B=8: the batch's loss and gradients equal the
  mean over its eight sequences (a property at any size), and its loss is the
  bf16 step's within the bars.
"""

import numpy as np
import pytest

import oracle
from oracle import gpt2 as og
import autograd_transformer_amd as tt
from autograd_transformer_amd import synthetic as syn
from tests.conftest import rel_l2
from tests.gpu_util import (dev, host, empty, zeros, tol, sync, split_key_bias, KEY_BIAS_NOISE,
                            check_post_adamw)

pytestmark = pytest.mark.gpu

HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1)
SHAPE = syn.ModelShape(n_layer=2, n_embd=128, n_head=2, vocab=97, block_size=80)
CFG = og.GPTConfig(n_layer=2, n_embd=128, n_head=2, vocab=97, block_size=80)
B, T = 3, 77


def _model(ctx, params, mode="fp16"):
    m = tt.Model(ctx, L=SHAPE.n_layer, C=SHAPE.n_embd, NH=SHAPE.n_head, V=SHAPE.vocab,
                 T_max=SHAPE.block_size, B_max=B, mode=mode, V_pad=128)
    m.load(params)
    return m


def _data(seed):
    params = syn.gpt2_params(SHAPE, seed=seed, w_std=0.05, bias_std=0.05, ln_std=0.1)
    tok, tgt = syn.gpt2_tokens(B, T, SHAPE.vocab, seed=seed)
    return params, tok, tgt


def test_fp16_step_at_fixed_scale_matches_oracle():
    params, tok, tgt = _data(51)
    p64 = {k: v.astype(np.float64) for k, v in params.items()}
    scale = 1024.0
    l_ref, g_ref = og.model_fwd_bwd(p64, tok, tgt, CFG, "fp16", loss_scale=scale)
    ctx = tt.Context(arena_bytes=1 << 30)
    model = _model(ctx, params)
    assert tt.tt_model_loss_scale_get(ctx, model) == (65536.0, 0, 0)   # the default
    tt.tt_model_loss_scale_set(ctx, model, scale)
    loss = empty((1,))
    tt.tt_model_fwd_bwd(ctx, model, B, T, dev(tok, "i32"), dev(tgt, "i32"), loss)
    sync()
    assert abs(host(loss)[0] - l_ref) / l_ref <= tol("fp16")
    errs, kb = {}, {}
    for k in g_ref:
        got = host(model.tensor(k, "g"))
        got = got[:SHAPE.vocab] if k == "wte" else got
        rest, rest_ref, key = split_key_bias(k, got, g_ref[k], SHAPE.n_embd)
        errs[k] = rel_l2(rest, rest_ref)
        if key is not None:
            kb[k] = np.linalg.norm(key) / np.linalg.norm(rest_ref)
    bad = {k: e for k, e in errs.items() if not e <= tol("fp16")}
    assert not bad, bad
    assert max(kb.values()) <= KEY_BIAS_NOISE["fp16"], kb
    tt.tt_model_adamw(ctx, model, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"], 1)
    sync()
    for k in g_ref:
        w_ref, _, _ = oracle.adamw_update(p64[k], g_ref[k], 0, 0, t=1, **HP)
        got = host(model.tensor(k, "w"))
        got = got[:SHAPE.vocab] if k == "wte" else got
        rms = np.linalg.norm(g_ref[k]) / np.sqrt(g_ref[k].size)
        gk = g_ref[k].copy()
        if k.endswith("b_qkv"):
            gk[SHAPE.n_embd:2 * SHAPE.n_embd] = 0.0
        check_post_adamw(got, p64[k], gk, w_ref, HP["lr"], HP["wd"], tol("fp16"), rms)
    # the shadow is binary16 of the master weights
    wl = host(model.tensor("h1.w_fc", "w_lowp"))
    assert np.array_equal(wl, oracle.round_fp16(host(model.tensor("h1.w_fc", "w"))))
    assert tt.tt_model_loss_scale_get(ctx, model) == (scale, 1, 0)
    model.close()
    ctx.close()


def test_fp16_overflow_drops_the_step_and_halves_the_scale():
    params, tok, tgt = _data(52)
    p64 = {k: v.astype(np.float64) for k, v in params.items()}
    zeros64 = {k: np.zeros_like(v) for k, v in p64.items()}
    ctx = tt.Context(arena_bytes=1 << 30)
    model = _model(ctx, params)
    tok_d, tgt_d = dev(tok, "i32"), dev(tgt, "i32")
    loss, flag = empty((1,)), zeros((1,), "i32")
    # 2**40 / N puts the label's dlogit far past the largest binary16
    big = 2.0 ** 40
    ref = og.train_step_scaled(p64, zeros64, dict(zeros64), 1, tok, tgt, CFG, big, 0, **HP)
    assert ref[-1] is True                      # the oracle drops this step too
    tt.tt_model_loss_scale_set(ctx, model, big)
    before = {k: host(model.tensor(k, "w")) for k in model.names}
    tt.tt_train_step(ctx, model, B, T, tok_d, tgt_d, HP["lr"], HP["beta1"], HP["beta2"],
                     HP["eps"], HP["wd"], 1, loss, flag)
    sync()
    assert int(host(flag)[0]) == 1
    for k in model.names:
        assert np.array_equal(host(model.tensor(k, "w")), before[k]), k
        assert not np.any(host(model.tensor(k, "m"))), k
    assert tt.tt_model_loss_scale_get(ctx, model) == (ref[5], 0, 1) == (big / 2, 0, 1)
    # a representable scale: the next step trains, as the oracle's does
    scale = 512.0
    ref = og.train_step_scaled(p64, zeros64, dict(zeros64), 1, tok, tgt, CFG, scale, 0, **HP)
    assert ref[-1] is False
    tt.tt_model_loss_scale_set(ctx, model, scale)
    tt.tt_train_step(ctx, model, B, T, tok_d, tgt_d, HP["lr"], HP["beta1"], HP["beta2"],
                     HP["eps"], HP["wd"], 1, loss, flag)
    sync()
    assert int(host(flag)[0]) == 0
    assert abs(host(loss)[0] - ref[0]) / ref[0] <= tol("fp16")
    for k in ("h0.w_qkv", "h1.w_fcp", "wte"):
        got = host(model.tensor(k, "m"))
        got = got[:SHAPE.vocab] if k == "wte" else got
        assert rel_l2(got, ref[3][k]) <= tol("fp16"), k
    assert tt.tt_model_loss_scale_get(ctx, model) == (scale, 1, 0)
    model.close()
    ctx.close()


def test_fp16_scale_schedule_follows_the_oracle():
    """interval 2, growth 2: the device counters step exactly like
    oracle.loss_scale_update, with one forced overflow in the middle."""
    params, tok, tgt = _data(53)
    ctx = tt.Context(arena_bytes=1 << 30)
    model = _model(ctx, params)
    tok_d, tgt_d = dev(tok, "i32"), dev(tgt, "i32")
    loss, flag = empty((1,)), zeros((1,), "i32")
    s, g = 64.0, 0
    tt.tt_model_loss_scale_set(ctx, model, s, 2, 2.0, 0.5)
    skipped = 0
    for step in range(1, 8):
        if step == 4:     # force an overflow at this step
            tt.tt_model_loss_scale_set(ctx, model, 2.0 ** 40, 2, 2.0, 0.5)
            s, g, skipped = 2.0 ** 40, 0, 0
        if step == 5:     # back to a representable scale (counters restart)
            tt.tt_model_loss_scale_set(ctx, model, 32.0, 2, 2.0, 0.5)
            s, g, skipped = 32.0, 0, 0
        tt.tt_train_step(ctx, model, B, T, tok_d, tgt_d, HP["lr"], HP["beta1"], HP["beta2"],
                         HP["eps"], HP["wd"], step, loss, flag)
        sync()
        over = bool(host(flag)[0])
        assert over == (step == 4), step
        s, g = oracle.loss_scale_update(s, g, over, interval=2, growth=2.0, backoff=0.5)
        skipped += over
        assert tt.tt_model_loss_scale_get(ctx, model) == (s, g, skipped), step
    model.close()
    ctx.close()


def test_fp16_refuses_decoding():
    params, _, _ = _data(54)
    ctx = tt.Context(arena_bytes=1 << 30)
    model = _model(ctx, params)
    with pytest.raises(tt.TTError, match="decoding"):
        tt.KVCache(ctx, model, 1)
    bf = _model(ctx, params, mode="bf16")
    with pytest.raises(tt.TTError, match="TT_FP16"):
        tt.tt_model_loss_scale_set(ctx, bf, 1024.0)
    model.close()
    bf.close()
    ctx.close()


@pytest.fixture(scope="module")
def gpt2_124m_fp16():
    shape = syn.GPT2_124M
    ctx = tt.Context(arena_bytes=24 << 30)
    model = tt.Model(ctx, L=12, C=768, NH=12, V=50257, T_max=1024, B_max=8, mode="fp16",
                     V_pad=50304)
    params = syn.gpt2_params(shape, seed=3)
    yield ctx, model, params
    model.close()
    ctx.close()


def test_gpt2_124m_fp16_batch_is_mean_of_sequences(gpt2_124m_fp16):
    """B=8, T=1024 in fp16 at a fixed scale: the batch's loss and gradients
    equal the mean of its eight single-sequence steps."""
    ctx, model, params = gpt2_124m_fp16
    model.load(params)
    tt.tt_model_loss_scale_set(ctx, model, 32768.0)
    tok, tgt = syn.gpt2_tokens(8, 1024, seed=41)
    loss = empty((1,))
    tt.tt_model_fwd_bwd(ctx, model, 8, 1024, dev(tok, "i32"), dev(tgt, "i32"), loss)
    sync()
    lB = host(loss)[0]
    gB = {k: host(model.tensor(k, "g")) for k in model.names}
    assert all(np.all(np.isfinite(v)) for v in gB.values())
    acc = {k: np.zeros_like(v) for k, v in gB.items()}
    lsum = 0.0
    for b in range(8):
        tt.tt_model_fwd_bwd(ctx, model, 1, 1024, dev(tok[b:b + 1], "i32"),
                            dev(tgt[b:b + 1], "i32"), loss)
        sync()
        lsum += host(loss)[0]
        for k in acc:
            acc[k] += host(model.tensor(k, "g"))
    assert abs(lB - lsum / 8) / lB <= 1e-5
    errs = {k: rel_l2(gB[k], acc[k] / 8) for k in acc}
    bad = {k: e for k, e in errs.items() if not e <= tol("fp16")}
    assert not bad, bad
    assert abs(lB - (np.log(50257) + 0.02 ** 2 * 768 / 2)) < 0.1
