"""Global-norm gradient clipping and safetensors checkpoints.

* tt_clip_grad_norm on flat buffers (ragged lengths, both sides of the
  threshold) and tt_model_clip_grad_norm between the backward and AdamW of a
  small model, against oracle.clip_grad_norm applied to the oracle's
  gradients (norm, clipped gradients and the AdamW moments that follow);
* tt_model_save / tt_model_load_state: a bit-exact round trip of weights,
  moments and step; the file read by the safetensors library (an independent
  reader of the format) with the GPT-2 tensor names and shapes; a
  weights-only file written by that library loaded through the C ABI; a run
  resumed from a checkpoint against the same run uninterrupted; malformed
  files rejected.
"""

import numpy as np
import pytest

import oracle
from oracle import gpt2 as og
import autograd_transformer_amd as tt
from autograd_transformer_amd import synthetic as syn
from tests.conftest import rel_l2
from tests.gpu_util import dev, host, empty, tol, sync

pytestmark = pytest.mark.gpu

HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1)
SHAPE = syn.ModelShape(n_layer=2, n_embd=128, n_head=2, vocab=97, block_size=80)
CFG = og.GPTConfig(n_layer=2, n_embd=128, n_head=2, vocab=97, block_size=80)


def _model(ctx, mode, params, B=3):
    m = tt.Model(ctx, L=SHAPE.n_layer, C=SHAPE.n_embd, NH=SHAPE.n_head, V=SHAPE.vocab,
                 T_max=SHAPE.block_size, B_max=B, mode=mode, V_pad=128)
    m.load(params)
    return m


@pytest.mark.parametrize("n,scale,max_norm", [
    (2, 1.0, 1.0),            # [3, 4]: norm 5, clipped to [0.6, 0.8]
    (1_000_003, 1.0, 10.0),   # clipped, ragged tail
    (4096, 1e-3, 10.0),       # below the threshold: untouched
    (7, 2.0, 0.5),
])
def test_clip_grad_norm_buffer(n, scale, max_norm):
    rng = np.random.default_rng(n)
    g = np.array([3.0, 4.0]) if n == 2 else rng.standard_normal(n) * scale
    g = g.astype(np.float32)
    ctx = tt.Context(arena_bytes=1 << 26)
    gd, norm = dev(g), empty((1,))
    tt.tt_clip_grad_norm(ctx, gd, max_norm, norm)
    sync()
    ref, total = oracle.clip_grad_norm({"g": g}, max_norm)
    assert abs(host(norm)[0] - total) <= 1e-6 * total
    got = host(gd)
    if max_norm / (total + 1e-6) >= 1.0:
        assert np.array_equal(got, g.astype(np.float64))
    else:
        assert rel_l2(got, ref["g"]) <= 1e-6
        assert abs(np.linalg.norm(got) - max_norm) <= 1e-5 * max_norm
    if n == 2:
        np.testing.assert_allclose(got, [0.6, 0.8], rtol=1e-6)
    ctx.close()


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_model_step_with_clipping(mode):
    """fwd_bwd -> clip (max norm a quarter of the gradient's) -> AdamW."""
    B, T = 3, 77
    params = syn.gpt2_params(SHAPE, seed=41, w_std=0.05, bias_std=0.05, ln_std=0.1)
    tok, tgt = syn.gpt2_tokens(B, T, SHAPE.vocab, seed=41)
    p64 = {k: v.astype(np.float64) for k, v in params.items()}
    l_ref, g_ref = og.model_fwd_bwd(p64, tok, tgt, CFG, mode)
    total_ref = np.sqrt(sum(float(np.sum(v * v)) for v in g_ref.values()))
    max_norm = 0.25 * total_ref
    g_clip, total = oracle.clip_grad_norm(g_ref, max_norm)
    ctx = tt.Context(arena_bytes=1 << 30)
    model = _model(ctx, mode, params, B)
    loss, norm = empty((1,)), empty((1,))
    tt.tt_model_fwd_bwd(ctx, model, B, T, dev(tok, "i32"), dev(tgt, "i32"), loss)
    tt.tt_model_clip_grad_norm(ctx, model, max_norm, norm)
    sync()
    assert abs(host(norm)[0] - total) <= tol(mode) * total
    got_total = np.sqrt(sum(float(np.sum(host(model.tensor(k, "g")) ** 2)) for k in model.names))
    assert abs(got_total - max_norm) <= 1e-5 * max_norm
    gq = {k: host(model.tensor(k, "g")) for k in model.names}
    for k in g_clip:
        got = gq[k][:SHAPE.vocab] if k == "wte" else gq[k]
        if k.endswith("b_qkv"):
            continue   # key third is exactly zero in the oracle; checked elsewhere
        assert rel_l2(got, g_clip[k]) <= tol(mode), k
    tt.tt_model_adamw(ctx, model, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"], 1)
    sync()
    for k in ("wte", "h0.w_qkv", "h1.w_fcp", "h1.b_fc", "lnf_g"):
        _, m_ref, v_ref = oracle.adamw_update(p64[k], g_clip[k], 0, 0, t=1, **HP)
        m_got = host(model.tensor(k, "m"))
        v_got = host(model.tensor(k, "v"))
        if k == "wte":
            m_got, v_got = m_got[:SHAPE.vocab], v_got[:SHAPE.vocab]
        assert rel_l2(m_got, m_ref) <= tol(mode), k
        assert rel_l2(v_got, v_ref) <= 2 * tol(mode), k
    model.close()
    ctx.close()


def _train(ctx, model, tok_d, tgt_d, B, T, t):
    loss = empty((1,))
    tt.tt_model_fwd_bwd(ctx, model, B, T, tok_d, tgt_d, loss)
    tt.tt_model_clip_grad_norm(ctx, model, 1.0)
    tt.tt_model_adamw(ctx, model, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"], t)
    sync()
    return float(host(loss)[0])


def _state(model):
    return {(k, w): host(model.tensor(k, w)) for k in model.names for w in ("w", "m", "v")}


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_checkpoint_round_trip_and_resume(mode, tmp_path):
    B, T = 2, 64
    params = syn.gpt2_params(SHAPE, seed=42, w_std=0.05, bias_std=0.05, ln_std=0.1)
    tok, tgt = syn.gpt2_tokens(B, T, SHAPE.vocab, seed=42)
    tok_d, tgt_d = dev(tok, "i32"), dev(tgt, "i32")
    ctx = tt.Context(arena_bytes=1 << 30)
    a = _model(ctx, mode, params, B)
    _train(ctx, a, tok_d, tgt_d, B, T, 1)
    _train(ctx, a, tok_d, tgt_d, B, T, 2)
    path = str(tmp_path / "ckpt.safetensors")
    tt.tt_model_save(ctx, a, path, 2)
    b = _model(ctx, mode, syn.gpt2_params(SHAPE, seed=7), B)
    assert tt.tt_model_load_state(ctx, b, path) == 2
    sync()
    sa, sb = _state(a), _state(b)
    for key in sa:
        assert np.array_equal(sa[key], sb[key]), key
    if mode == "bf16":
        for k in ("wte", "h1.w_fc"):
            assert np.array_equal(host(b.tensor(k, "w_lowp")),
                                  oracle.round_bf16(host(b.tensor(k, "w"))))
    # resumed run == uninterrupted run (up to the order of atomic additions)
    la = _train(ctx, a, tok_d, tgt_d, B, T, 3)
    lb = _train(ctx, b, tok_d, tgt_d, B, T, 3)
    assert abs(la - lb) <= 1e-6 * abs(la)
    sa, sb = _state(a), _state(b)
    for key in sa:
        assert rel_l2(sb[key], sa[key]) <= 1e-4, key
    a.close()
    b.close()
    ctx.close()


def _hf_names():
    names = {"wte": "wte.weight", "wpe": "wpe.weight", "lnf_g": "ln_f.weight",
             "lnf_b": "ln_f.bias"}
    per = dict(ln1_g="ln_1.weight", ln1_b="ln_1.bias", w_qkv="attn.c_attn.weight",
               b_qkv="attn.c_attn.bias", w_proj="attn.c_proj.weight", b_proj="attn.c_proj.bias",
               ln2_g="ln_2.weight", ln2_b="ln_2.bias", w_fc="mlp.c_fc.weight", b_fc="mlp.c_fc.bias",
               w_fcp="mlp.c_proj.weight", b_fcp="mlp.c_proj.bias")
    for l in range(SHAPE.n_layer):
        for k, v in per.items():
            names[f"h{l}.{k}"] = f"h.{l}.{v}"
    return names


def test_checkpoint_file_read_and_written_by_safetensors(tmp_path):
    from safetensors.numpy import load_file, save_file
    B, T = 2, 32
    params = syn.gpt2_params(SHAPE, seed=43, w_std=0.05, bias_std=0.05, ln_std=0.1)
    tok, tgt = syn.gpt2_tokens(B, T, SHAPE.vocab, seed=43)
    ctx = tt.Context(arena_bytes=1 << 30)
    a = _model(ctx, "bf16", params, B)
    _train(ctx, a, dev(tok, "i32"), dev(tgt, "i32"), B, T, 1)
    path = str(tmp_path / "a.safetensors")
    tt.tt_model_save(ctx, a, path, 1)
    f = load_file(path)
    names = _hf_names()
    assert set(f) == ({v for v in names.values()} | {"adam_m." + v for v in names.values()}
                      | {"adam_v." + v for v in names.values()} | {"adam_step"})
    assert f["adam_step"].dtype == np.int64 and f["adam_step"].tolist() == [1]
    for ours, hf in names.items():
        want = host(a.tensor(ours, "w"))
        if ours == "wte":
            want = want[:SHAPE.vocab]
        assert f[hf].dtype == np.float32 and f[hf].shape == want.shape, hf
        assert np.array_equal(f[hf].astype(np.float64), want), hf
        m = host(a.tensor(ours, "m"))
        assert np.array_equal(f["adam_m." + hf].astype(np.float64),
                              m[:SHAPE.vocab] if ours == "wte" else m), hf
    # a weights-only file from the safetensors writer: moments start at zero
    w2 = syn.gpt2_params(SHAPE, seed=44, w_std=0.05)
    p2 = str(tmp_path / "b.safetensors")
    save_file({names[k]: np.ascontiguousarray(v, np.float32) for k, v in w2.items()}, p2)
    assert tt.tt_model_load_state(ctx, a, p2) == 0
    sync()
    for k, v in w2.items():
        got = host(a.tensor(k, "w"))
        if k == "wte":
            assert np.all(got[SHAPE.vocab:] == 0)
            got = got[:SHAPE.vocab]
        assert np.array_equal(got, v.astype(np.float64)), k
        assert not np.any(host(a.tensor(k, "m"))) and not np.any(host(a.tensor(k, "v"))), k
    a.close()
    ctx.close()


def test_checkpoint_rejects_bad_files(tmp_path):
    from safetensors.numpy import save_file
    ctx = tt.Context(arena_bytes=1 << 28)
    a = _model(ctx, "f32", syn.gpt2_params(SHAPE, seed=45))
    names = _hf_names()
    with pytest.raises(tt.TTError):
        tt.tt_model_load_state(ctx, a, str(tmp_path / "missing.safetensors"))
    junk = tmp_path / "junk.safetensors"
    junk.write_bytes(b"\xff" * 64)
    with pytest.raises(tt.TTError):
        tt.tt_model_load_state(ctx, a, str(junk))
    w = {names[k]: np.ascontiguousarray(v, np.float32)
         for k, v in syn.gpt2_params(SHAPE, seed=46).items()}
    bad_shape = dict(w)
    bad_shape["h.1.mlp.c_fc.weight"] = np.zeros((4 * SHAPE.n_embd, SHAPE.n_embd), np.float32)
    save_file(bad_shape, str(tmp_path / "shape.safetensors"))
    with pytest.raises(tt.TTError, match="c_fc"):
        tt.tt_model_load_state(ctx, a, str(tmp_path / "shape.safetensors"))
    missing = dict(w)
    del missing["ln_f.bias"]
    save_file(missing, str(tmp_path / "lack.safetensors"))
    with pytest.raises(tt.TTError, match="ln_f.bias"):
        tt.tt_model_load_state(ctx, a, str(tmp_path / "lack.safetensors"))
    half = {k: v.astype(np.float16) for k, v in w.items()}
    save_file(half, str(tmp_path / "f16.safetensors"))
    with pytest.raises(tt.TTError, match="dtype"):
        tt.tt_model_load_state(ctx, a, str(tmp_path / "f16.safetensors"))
    a.close()
    ctx.close()
