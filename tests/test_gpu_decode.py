"""Greedy generation with the key/value cache against the oracle.

* tt_argmax: bit-exact against the oracle's rule (lowest index on ties, first
  NaN) on the same values, bf16 and fp32, vector and scalar row layouts;
* prefill + decode of a small model in both modes: every step's logits
  against the oracle's full-sequence forward over the tokens the GPU chose
  (teacher forcing: causality makes the two the same computation), the GPU's
  token equal to the argmax of its own logits, and to the oracle's argmax
  wherever the oracle's top-two margin exceeds the observed error; the
  decode steps replay one captured HIP graph, and the same steps run
  eagerly match every replay bit for bit;
* the full-size GPT-2 124M model (bf16): a decode step after a prefill gives
  the logits a prefill over the longer sequence gives (a property that holds
  at any size).
"""

import numpy as np
import pytest

import oracle
from oracle import gpt2 as og
import autograd_transformer_amd as tt
from autograd_transformer_amd import synthetic as syn
from tests.conftest import rel_l2
from tests.gpu_util import dev, host, empty, lowp, tol, sync

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = tt.Context(arena_bytes=4 << 30)
    yield c
    c.close()


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("NVL", [(37, 1000, 1000), (8, 50257, 50304), (6, 13, 13), (5, 101, 103)])
def test_argmax_matches_oracle_rule(ctx, mode, NVL):
    N, V, ld = NVL
    z = syn.normal(300 + V, (N, ld), 3.0)
    if mode == "bf16":
        z = syn.bf16_exact(z)
    z[:, V:] = 1e30                       # columns past V must be ignored
    z[0, [V // 3, V // 2]] = 50.0          # tie: the lower index wins
    if N > 1:
        z[1, :V] = 2.0                     # all equal
    if N > 2:
        z[2, [V // 4, V - 1]] = np.nan     # first NaN
    if N > 3:
        z[3, :V] = -np.inf
    if N > 4:
        z[4, V - 1] = 60.0                 # maximum in the ragged tail
    out = empty((N,), "i32")
    tt.tt_argmax(ctx, mode, N, V, ld, dev(z, lowp(mode)), out)
    sync()
    got = host(out).astype(np.int64)
    want = oracle.argmax_rows(z[:, :V])
    assert np.array_equal(got, want), (got, want)


def _small(mode, seed=5):
    shape = syn.ModelShape(2, 128, 2, 997, 64)
    params = syn.gpt2_params(shape, seed=seed, w_std=0.1, bias_std=0.02, ln_std=0.1)
    cfg = og.GPTConfig(n_layer=2, n_embd=128, n_head=2, vocab=997, block_size=64)
    return shape, params, cfg


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_prefill_and_decode_small_model_against_oracle(ctx, mode):
    shape, params, cfg = _small(mode)
    B, T0, steps = 3, 7, 9
    model = tt.Model(ctx, L=2, C=128, NH=2, V=997, T_max=64, B_max=4, mode=mode, V_pad=1024)
    model.load(params)
    cache = tt.KVCache(ctx, model, 4)
    prompt = np.random.default_rng(8).integers(0, 997, size=(B, T0)).astype(np.int32)
    nxt = empty((B,), "i32")
    lg = empty((B, 997), lowp(mode))
    tt.tt_model_prefill(ctx, model, cache, B, T0, dev(prompt, "i32"), lg, nxt)
    sync()
    seq = [prompt]
    logits = [host(lg)]
    toks = [host(nxt).astype(np.int64)]
    for j in range(steps):
        tok_d = dev(toks[-1].astype(np.int32), "i32")
        tt.tt_model_decode(ctx, model, cache, B, T0 + j, tok_d, lg, nxt)
        sync()
        logits.append(host(lg))
        toks.append(host(nxt).astype(np.int64))
    seq = np.concatenate([prompt] + [t[:, None] for t in toks[:-1]], axis=1)
    p64 = {k: v.astype(np.float64) for k, v in params.items()}
    z = og.model_logits(p64, seq, cfg, mode)            # [B, T0 + steps, V]
    for j in range(steps + 1):
        ref = z[:, T0 - 1 + j]
        got = logits[j]
        assert rel_l2(got, ref) <= tol(mode), (j, rel_l2(got, ref))
        assert np.array_equal(toks[j], oracle.argmax_rows(got)), j
        err = np.abs(got - ref).max()
        top2 = np.sort(ref, axis=-1)[:, -2:]
        clear = (top2[:, 1] - top2[:, 0]) > 2 * err + 1e-12
        assert np.array_equal(toks[j][clear], oracle.argmax_rows(ref)[clear]), j
    # The steps above replayed one captured graph; run them again eagerly
    # (profiling mode launches every kernel on the context's stream) and
    # compare every step bit for bit.
    ctx.profile(True)
    tt.tt_model_prefill(ctx, model, cache, B, T0, dev(prompt, "i32"), lg, nxt)
    sync()
    assert np.array_equal(host(lg), logits[0])
    for j in range(steps):
        tt.tt_model_decode(ctx, model, cache, B, T0 + j, dev(toks[j].astype(np.int32), "i32"), lg,
                           nxt)
        sync()
        assert np.array_equal(host(lg), logits[j + 1]), j
        assert np.array_equal(host(nxt).astype(np.int64), toks[j + 1]), j
    ctx.profile_report()
    ctx.profile(False)
    cache.close()
    model.close()


def test_decode_matches_longer_prefill_gpt2_124m():
    """After a prefill of T0 tokens, decoding token x at position T0 gives the
    logits that a prefill of the T0 + 1 tokens gives at its last position."""
    params = syn.gpt2_params(syn.GPT2_124M, seed=3)
    c = tt.Context(arena_bytes=24 << 30)
    model = tt.Model(c, L=12, C=768, NH=12, V=50257, T_max=1024, B_max=8, mode="bf16",
                     V_pad=50304)
    model.load(params)
    cache = tt.KVCache(c, model, 8)
    B, T0 = 8, 600
    tok = np.random.default_rng(21).integers(0, 50257, size=(B, T0 + 1)).astype(np.int32)
    nxt = empty((B,), "i32")
    la, lb = empty((B, 50257), "bf16"), empty((B, 50257), "bf16")
    tt.tt_model_prefill(c, model, cache, B, T0, dev(tok[:, :T0], "i32"), la, nxt)
    tt.tt_model_decode(c, model, cache, B, T0, dev(tok[:, T0].copy(), "i32"), la, nxt)
    sync()
    dec, dec_tok = host(la), host(nxt).astype(np.int64)
    tt.tt_model_prefill(c, model, cache, B, T0 + 1, dev(tok, "i32"), lb, nxt)
    sync()
    full = host(lb)
    assert rel_l2(dec, full) <= 2e-2, rel_l2(dec, full)
    assert np.array_equal(dec_tok, oracle.argmax_rows(dec))
    err = np.abs(dec - full).max()
    top2 = np.sort(full, axis=-1)[:, -2:]
    clear = (top2[:, 1] - top2[:, 0]) > 2 * err
    assert np.array_equal(dec_tok[clear], oracle.argmax_rows(full)[clear])
    cache.close()
    model.close()
    c.close()
