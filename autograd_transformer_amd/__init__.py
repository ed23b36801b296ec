"""MI355X-native GPT-2 training step: Python binding of the libtt C ABI.

The functions here have the names of the C entry points (include/tt.h) and
only marshal arguments: torch tensors become device pointers, results come
back as tensors the caller passed in.  PyTorch provides device memory and the
stream; every step of the computation runs in libtt's HIP kernels.  Importing
the package does not load the library; the first call does, and raises if it
was not built.
"""

import ctypes as _C
import os

from . import _lib as _L

TT_F32, TT_BF16, TT_FP16 = 0, 1, 2
TT_EPI_NONE, TT_EPI_GELU, TT_EPI_RESIDUAL = 0, 1, 2

STATUS = {0: "TT_OK", -1: "TT_EINVAL", -2: "TT_ENOMEM", -3: "TT_EHIP", -4: "TT_ESTALE",
          -5: "TT_ENONFINITE", -6: "TT_EUNSUPPORTED", -7: "TT_ERANGE"}


class TTError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def lib():
    return _L.load()


def _ptr(t):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _mode(m):
    if m in (TT_F32, TT_BF16, TT_FP16):
        return m
    return {"f32": TT_F32, "bf16": TT_BF16, "fp16": TT_FP16}[m]


class Context:
    """A libtt context bound to a device and a HIP stream (torch's current one
    by default), owning an HBM arena of ``arena_bytes``."""

    def __init__(self, arena_bytes, device=0, stream=None):
        import torch
        torch.cuda.set_device(device)
        if stream is None:
            stream = torch.cuda.current_stream(device)
        self.stream = stream
        self.device = device
        h = _C.c_void_p()
        rc = lib().tt_ctx_create(device, stream.cuda_stream, int(arena_bytes), None, _C.byref(h))
        if rc != 0:
            raise TTError(rc, lib().tt_strerror(rc).decode())
        self.handle = h

    def check(self, rc):
        if rc != 0:
            raise TTError(rc, lib().tt_ctx_last_error(self.handle).decode())
        return rc

    def close(self):
        if getattr(self, "handle", None):
            lib().tt_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def sync(self):
        return self.check(lib().tt_ctx_sync(self.handle))

    def alloc(self, nbytes, align=256):
        p = _C.c_void_p()
        self.check(lib().tt_ctx_alloc(self.handle, int(nbytes), int(align), _C.byref(p)))
        return p.value

    def mark(self):
        return self.check(lib().tt_ctx_mark(self.handle))

    def reset(self):
        return self.check(lib().tt_ctx_reset(self.handle))

    def profile(self, enable):
        """Start (clearing earlier records) or stop per-kernel event timing."""
        return self.check(lib().tt_ctx_profile(self.handle, 1 if enable else 0))

    def profile_report(self):
        """Per-kernel totals since profile(True): list of dicts with name,
        calls, ms, flops, bytes (algorithmic work of those launches)."""
        n = _C.c_int(0)
        self.check(lib().tt_ctx_profile_report(self.handle, None, _C.byref(n)))
        arr = (_L.tt_prof_entry * max(n.value, 1))()
        self.check(lib().tt_ctx_profile_report(self.handle, arr, _C.byref(n)))
        return [dict(name=e.name.decode(), calls=e.calls, ms=e.ms, flops=e.flops, bytes=e.bytes)
                for e in arr[: n.value]]

    def usage(self):
        u, c = _C.c_size_t(), _C.c_size_t()
        self.check(lib().tt_ctx_usage(self.handle, _C.byref(u), _C.byref(c)))
        return u.value, c.value


# ------------------------------------------------------------------ op level

def tt_linear_fwd(ctx, mode, M, K, N, X, W, b, Y, epilogue=TT_EPI_NONE, resid=None, preact=None):
    return ctx.check(lib().tt_linear_fwd(ctx.handle, _mode(mode), M, K, N, _ptr(X), _ptr(W),
                                         _ptr(b), _ptr(Y), epilogue, _ptr(resid), _ptr(preact)))


def tt_linear_bwd(ctx, mode, M, K, N, X, W, dY, dX=None, dW=None, db=None, accumulate_dX=False):
    return ctx.check(lib().tt_linear_bwd(ctx.handle, _mode(mode), M, K, N, _ptr(X), _ptr(W),
                                         _ptr(dY), _ptr(dX), _ptr(dW), _ptr(db),
                                         1 if accumulate_dX else 0))


def tt_layernorm_fwd(ctx, mode, N, C, eps, x, g, b, y, mean=None, rstd=None):
    return ctx.check(lib().tt_layernorm_fwd(ctx.handle, _mode(mode), N, C, eps, _ptr(x), _ptr(g),
                                            _ptr(b), _ptr(y), _ptr(mean), _ptr(rstd)))


def tt_layernorm_bwd(ctx, mode, N, C, x, mean, rstd, g, dy, dx, dg=None, db=None):
    return ctx.check(lib().tt_layernorm_bwd(ctx.handle, _mode(mode), N, C, _ptr(x), _ptr(mean),
                                            _ptr(rstd), _ptr(g), _ptr(dy), _ptr(dx), _ptr(dg),
                                            _ptr(db)))


def tt_layernorm_bwd_noalloc(ctx, mode, N, C, x, mean, rstd, g, dy, dx, dg=None, db=None):
    return ctx.check(lib().tt_layernorm_bwd_noalloc(ctx.handle, _mode(mode), N, C, _ptr(x),
                                                    _ptr(mean), _ptr(rstd), _ptr(g), _ptr(dy),
                                                    _ptr(dx), _ptr(dg), _ptr(db)))


def tt_gelu_fwd(ctx, mode, n, x, y):
    return ctx.check(lib().tt_gelu_fwd(ctx.handle, _mode(mode), n, _ptr(x), _ptr(y)))


def tt_gelu_bwd(ctx, mode, n, x, dy, dx):
    return ctx.check(lib().tt_gelu_bwd(ctx.handle, _mode(mode), n, _ptr(x), _ptr(dy), _ptr(dx)))


def tt_attn_fwd(ctx, mode, B, T, NH, hs, qkv, out, lse):
    return ctx.check(lib().tt_attn_fwd(ctx.handle, _mode(mode), B, T, NH, hs, _ptr(qkv),
                                       _ptr(out), _ptr(lse)))


def tt_attn_bwd(ctx, mode, B, T, NH, hs, qkv, out, lse, dout, dqkv):
    return ctx.check(lib().tt_attn_bwd(ctx.handle, _mode(mode), B, T, NH, hs, _ptr(qkv),
                                       _ptr(out), _ptr(lse), _ptr(dout), _ptr(dqkv)))


def tt_ce_fwdbwd(ctx, mode, N, V, ld, logits, targets, loss, grad_scale=0.0):
    return ctx.check(lib().tt_ce_fwdbwd(ctx.handle, _mode(mode), N, V, ld, _ptr(logits),
                                        _ptr(targets), _ptr(loss), grad_scale))


def tt_embed_fwd(ctx, B, T, C, V, tok, wte, wpe, x0):
    return ctx.check(lib().tt_embed_fwd(ctx.handle, B, T, C, V, _ptr(tok), _ptr(wte), _ptr(wpe),
                                        _ptr(x0)))


def tt_embed_bwd(ctx, B, T, C, V, tok, dx0, dwte=None, dwpe=None):
    return ctx.check(lib().tt_embed_bwd(ctx.handle, B, T, C, V, _ptr(tok), _ptr(dx0), _ptr(dwte),
                                        _ptr(dwpe)))


def tt_adamw_step(ctx, params, lr, beta1, beta2, eps, wd, t):
    """params: list of dicts with tensors w, g, m, v, optional w_lowp, optional wd_mult."""
    arr = (_L.tt_param * len(params))()
    for i, p in enumerate(params):
        arr[i].w, arr[i].g, arr[i].m, arr[i].v = (_ptr(p[k]) for k in ("w", "g", "m", "v"))
        arr[i].w_lowp = _ptr(p.get("w_lowp"))
        arr[i].n = p["w"].numel()
        arr[i].wd_mult = float(p.get("wd_mult", 1.0))
    return ctx.check(lib().tt_adamw_step(ctx.handle, arr, len(params), lr, beta1, beta2, eps, wd, t))


def tt_sgd_step(ctx, w, g, lr):
    return ctx.check(lib().tt_sgd_step(ctx.handle, _ptr(w), _ptr(g), w.numel(), lr))


def tt_cast_bf16(ctx, src, dst):
    return ctx.check(lib().tt_cast_bf16(ctx.handle, src.numel(), _ptr(src), _ptr(dst)))


# ------------------------------------------------------------------ composites

BLOCK_TENSORS = list(_L._BLOCK_W)


def _block_cfg(B, T, C, NH, F, mode, eps):
    return _L.tt_block_cfg(B, T, C, NH, F, _mode(mode), eps)


def _block_struct(cls, tensors):
    s = cls()
    for k in BLOCK_TENSORS:
        setattr(s, k, _ptr(tensors[k]))
    return s


class BlockSaved:
    def __init__(self, ctx, B, T, C, NH, F, mode, eps=1e-5):
        self.ctx = ctx
        self.cfg = _block_cfg(B, T, C, NH, F, mode, eps)
        h = _C.c_void_p()
        ctx.check(lib().tt_block_saved_create(ctx.handle, _C.byref(self.cfg), _C.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            lib().tt_block_saved_destroy(self.handle)
            self.handle = None


def tt_block_fwd(ctx, saved, w, x, y):
    ws = _block_struct(_L.tt_block_w, w)
    return ctx.check(lib().tt_block_fwd(ctx.handle, _C.byref(saved.cfg), _C.byref(ws), _ptr(x),
                                        _ptr(y), saved.handle))


def tt_block_bwd(ctx, saved, w, dy, dx, grads):
    ws = _block_struct(_L.tt_block_w, w)
    gs = _block_struct(_L.tt_block_g, grads)
    return ctx.check(lib().tt_block_bwd(ctx.handle, _C.byref(saved.cfg), _C.byref(ws),
                                        saved.handle, _ptr(dy), _ptr(dx), _C.byref(gs)))


def tt_lmhead_ce_fwdbwd(ctx, mode, N, C, V, h, wte, targets, loss, dh, dwte):
    return ctx.check(lib().tt_lmhead_ce_fwdbwd(ctx.handle, _mode(mode), N, C, V, _ptr(h),
                                               _ptr(wte), _ptr(targets), _ptr(loss), _ptr(dh),
                                               _ptr(dwte)))


MODEL_LAYER_TENSORS = BLOCK_TENSORS


class Model:
    """GPT-2 parameters, gradients, AdamW moments and activations in the
    context's arena (tt_model_create)."""

    def __init__(self, ctx, L, C, NH, V, T_max, B_max, mode, V_pad=None, F=None, eps=1e-5):
        self.ctx = ctx
        F = 4 * C if F is None else F
        V_pad = V if V_pad is None else V_pad
        self.cfg = _L.tt_model_cfg(L, C, NH, F, V, V_pad, T_max, B_max, _mode(mode), eps)
        h = _C.c_void_p()
        ctx.check(lib().tt_model_create(ctx.handle, _C.byref(self.cfg), _C.byref(h)))
        self.handle = h
        n = _C.c_int(0)
        ctx.check(lib().tt_model_param_table(h, None, _C.byref(n)))
        self.table = (_L.tt_param * n.value)()
        ctx.check(lib().tt_model_param_table(h, self.table, _C.byref(n)))
        names = ["wte", "wpe"]
        for l in range(L):
            names += [f"h{l}.{k}" for k in MODEL_LAYER_TENSORS]
        names += ["lnf_g", "lnf_b"]
        self.names = names
        shapes = {"wte": (V_pad, C), "wpe": (T_max, C), "lnf_g": (C,), "lnf_b": (C,)}
        ls = dict(ln1_g=(C,), ln1_b=(C,), w_qkv=(C, 3 * C), b_qkv=(3 * C,), w_proj=(C, C),
                  b_proj=(C,), ln2_g=(C,), ln2_b=(C,), w_fc=(C, F), b_fc=(F,), w_fcp=(F, C),
                  b_fcp=(C,))
        for l in range(L):
            for k, s in ls.items():
                shapes[f"h{l}.{k}"] = s
        self.shapes = shapes
        ns, npar = _C.c_size_t(), _C.c_size_t()
        ctx.check(lib().tt_model_num_params(h, _C.byref(ns), _C.byref(npar)))
        self.n_slots, self.n_params = ns.value, npar.value

    def tensor(self, name, which="w"):
        """A torch view of one parameter's w / g / m / v (float32) or w_lowp (bf16)."""
        import torch
        i = self.names.index(name)
        p = self.table[i]
        addr = getattr(p, which)
        lowp = torch.float16 if self.cfg.mode == TT_FP16 else torch.bfloat16
        dtype = lowp if which == "w_lowp" else torch.float32
        return _tensor_view(addr, self.shapes[name], dtype, self.ctx.device)

    def load(self, params):
        """Copy host float32 arrays into the master weights, refresh the
        bf16 shadow and zero the AdamW moments."""
        import torch
        for k, v in params.items():
            t = self.tensor(k, "w")
            src = torch.as_tensor(v, dtype=torch.float32)
            if k == "wte" and src.shape[0] < t.shape[0]:
                t.zero_()
                t[: src.shape[0]].copy_(src)
            else:
                t.copy_(src.reshape(t.shape))
        torch.cuda.current_stream(self.ctx.device).synchronize()
        self.ctx.check(lib().tt_model_refresh_shadow(self.handle))

    def close(self):
        if getattr(self, "handle", None):
            lib().tt_model_destroy(self.handle)
            self.handle = None


def _tensor_view(addr, shape, dtype, device):
    """Wrap arena memory as a torch tensor without copying (memory stays owned
    by the libtt context)."""
    import torch
    n = 1
    for s in shape:
        n *= s
    esz = torch.tensor([], dtype=dtype).element_size()

    typestr = "<f4" if esz == 4 else ("<f2" if dtype == torch.float16 else "<u2")

    class _Arr:
        __cuda_array_interface__ = {
            "shape": (n,), "typestr": typestr,
            "data": (addr, False), "version": 2, "strides": None,
        }
    t = torch.as_tensor(_Arr(), device=f"cuda:{device}")
    if dtype == torch.bfloat16:
        t = t.view(torch.bfloat16)
    return t.view(*shape)


def tt_train_step(ctx, model, B, T, tok, targets, lr, beta1, beta2, eps, wd, t, loss,
                  nonfinite=None):
    return ctx.check(lib().tt_train_step(ctx.handle, model.handle, B, T, _ptr(tok), _ptr(targets),
                                         lr, beta1, beta2, eps, wd, t, _ptr(loss),
                                         _ptr(nonfinite)))


def tt_model_fwd_bwd(ctx, model, B, T, tok, targets, loss):
    return ctx.check(lib().tt_model_fwd_bwd(ctx.handle, model.handle, B, T, _ptr(tok),
                                            _ptr(targets), _ptr(loss)))


def tt_model_adamw(ctx, model, lr, beta1, beta2, eps, wd, t):
    return ctx.check(lib().tt_model_adamw(ctx.handle, model.handle, lr, beta1, beta2, eps, wd, t))


def tt_model_loss_scale_set(ctx, model, scale, interval=1000, growth=1.001, backoff=0.5):
    """Dynamic loss scaling policy and scale of a TT_FP16 model."""
    return ctx.check(lib().tt_model_loss_scale_set(ctx.handle, model.handle, scale, interval,
                                                   growth, backoff))


def tt_model_loss_scale_get(ctx, model):
    """(scale, clean steps since the last change, dropped steps) of a TT_FP16
    model; synchronises with the context's stream."""
    sc, good, skipped = _C.c_float(), _C.c_int(), _C.c_int()
    ctx.check(lib().tt_model_loss_scale_get(ctx.handle, model.handle, _C.byref(sc),
                                            _C.byref(good), _C.byref(skipped)))
    return sc.value, good.value, skipped.value


def tt_model_clip_grad_norm(ctx, model, max_norm, norm=None):
    """Scale every gradient of the model by max_norm / (norm + 1e-6) when that
    is below 1; norm (float32 [1] on the GPU, optional) receives the norm."""
    return ctx.check(lib().tt_model_clip_grad_norm(ctx.handle, model.handle, max_norm,
                                                   _ptr(norm)))


def tt_clip_grad_norm(ctx, g, max_norm, norm=None):
    """Global-norm clipping of one float32 gradient buffer in place."""
    return ctx.check(lib().tt_clip_grad_norm(ctx.handle, _ptr(g), g.numel(), max_norm,
                                             _ptr(norm)))


def tt_model_save(ctx, model, path, step):
    """Write weights, AdamW moments and the step count as a safetensors file."""
    return ctx.check(lib().tt_model_save(ctx.handle, model.handle, os.fsencode(path), step))


def tt_model_load_state(ctx, model, path):
    """Read a checkpoint written by tt_model_save (or a weights-only
    safetensors file with the same names); returns the stored step."""
    step = _C.c_int64(0)
    ctx.check(lib().tt_model_load_state(ctx.handle, model.handle, os.fsencode(path),
                                        _C.byref(step)))
    return step.value


def tt_mlp_step(ctx, x, labels, W1, b1, W2, b2, lr, loss, grads=None):
    """The tiny classifier's training step in one launch; weights updated in
    place, grads (optional dict W1/b1/W2/b2 of tensors) receive gradients."""
    N, I = x.shape
    H, C = W1.shape[1], W2.shape[1]
    g = grads or {}
    return ctx.check(lib().tt_mlp_step(ctx.handle, N, I, H, C, _ptr(x), _ptr(labels), _ptr(W1),
                                       _ptr(b1), _ptr(W2), _ptr(b2), lr, _ptr(loss),
                                       _ptr(g.get("W1")), _ptr(g.get("b1")), _ptr(g.get("W2")),
                                       _ptr(g.get("b2"))))


# ------------------------------------------------------------------ graph

class Graph:
    """Recorded-graph autograd (tt_graph): nodes are integer ids; leaves wrap
    caller float32 tensors, computed nodes live in the context's arena."""

    def __init__(self, ctx):
        self.ctx = ctx
        h = _C.c_void_p()
        ctx.check(lib().tt_graph_create(ctx.handle, _C.byref(h)))
        self.handle = h
        self._keep = []   # tensors the graph reads (leaves, targets)

    def _id(self, fn, *args):
        out = _C.c_int(-1)
        self.ctx.check(fn(self.handle, *args, _C.byref(out)))
        return out.value

    def leaf(self, data, grad=None):
        rows, cols = (1, data.shape[0]) if data.dim() == 1 else tuple(data.shape)
        self._keep += [data, grad]
        return self._id(lib().tt_graph_leaf, rows, cols, _ptr(data), _ptr(grad))

    def matmul(self, a, b):
        return self._id(lib().tt_graph_matmul, a, b)

    def add(self, a, b):
        return self._id(lib().tt_graph_add, a, b)

    def gelu(self, a):
        return self._id(lib().tt_graph_gelu, a)

    def softmax(self, a):
        return self._id(lib().tt_graph_softmax, a)

    def cross_entropy(self, logits, targets):
        self._keep.append(targets)
        return self._id(lib().tt_graph_cross_entropy, logits, _ptr(targets))

    def forward(self, node):
        return self.ctx.check(lib().tt_graph_forward(self.handle, node))

    def backward(self, loss):
        return self.ctx.check(lib().tt_graph_backward(self.handle, loss))

    def zero_grad(self):
        return self.ctx.check(lib().tt_graph_zero_grad(self.handle))

    def capture_sgd_step(self, loss, lr):
        """Record forward / zero_grad / backward / SGD as one HIP graph."""
        return self.ctx.check(lib().tt_graph_capture_sgd_step(self.handle, loss, lr))

    def step(self):
        """Replay the captured training step on the context's stream."""
        return self.ctx.check(lib().tt_graph_step(self.handle))

    def _tensor(self, node, which):
        import torch
        v, g = _C.c_void_p(), _C.c_void_p()
        r, c = _C.c_int(), _C.c_int()
        self.ctx.check(lib().tt_graph_tensor(self.handle, node, _C.byref(v), _C.byref(g),
                                             _C.byref(r), _C.byref(c)))
        addr = v.value if which == "value" else g.value
        if addr is None:
            return None
        return _tensor_view(addr, (r.value, c.value), torch.float32, self.ctx.device)

    def value(self, node):
        """A torch view of a node's value (valid while the arena holds it)."""
        return self._tensor(node, "value")

    def grad(self, node):
        return self._tensor(node, "grad")

    def close(self):
        if getattr(self, "handle", None):
            lib().tt_graph_destroy(self.handle)
            self.handle = None
        self._keep = []


# ------------------------------------------------------------------ inference

def tt_argmax(ctx, mode, N, V, ld, logits, out):
    """out[n] = argmax of logits[n, :V] (row stride ld), lowest index on ties."""
    return ctx.check(lib().tt_argmax(ctx.handle, _mode(mode), N, V, ld, _ptr(logits), _ptr(out)))


class KVCache:
    """Key/value cache of a model for up to B_max sequences (tt_kvcache)."""

    def __init__(self, ctx, model, B_max):
        self.ctx = ctx
        h = _C.c_void_p()
        ctx.check(lib().tt_kvcache_create(ctx.handle, model.handle, B_max, _C.byref(h)))
        self.handle = h
        self.B_max = B_max

    def close(self):
        if getattr(self, "handle", None):
            lib().tt_kvcache_destroy(self.handle)
            self.handle = None


def tt_model_prefill(ctx, model, cache, B, T, tok, logits, next_tok):
    return ctx.check(lib().tt_model_prefill(ctx.handle, model.handle, cache.handle, B, T,
                                            _ptr(tok), _ptr(logits), _ptr(next_tok)))


def tt_model_decode(ctx, model, cache, B, pos, tok, logits, next_tok):
    return ctx.check(lib().tt_model_decode(ctx.handle, model.handle, cache.handle, B, pos,
                                           _ptr(tok), _ptr(logits), _ptr(next_tok)))


# ------------------------------------------------------------------ probes

def tt_probe_mfma(ctx, waves_per_simd=2, accumulators=16, iters=20000):
    """Dense bf16 MFMA rate (TFLOP/s) with register operands only."""
    out = _C.c_double(0.0)
    ctx.check(lib().tt_probe_mfma(ctx.handle, waves_per_simd, accumulators, iters, _C.byref(out)))
    return out.value


def tt_probe_hbm(ctx, buf, copy=False):
    """Streaming HBM rate (GB/s) over a device tensor (read, or copy of its
    first half over its second)."""
    out = _C.c_double(0.0)
    nbytes = buf.numel() * buf.element_size()
    ctx.check(lib().tt_probe_hbm(ctx.handle, _ptr(buf), nbytes, 1 if copy else 0, _C.byref(out)))
    return out.value


def tt_probe_lds(ctx, mfma=False):
    """LDS fragment reads per clock per CU (bytes), alone or feeding MFMAs;
    returns (bytes_per_clk, tflops)."""
    b, t = _C.c_double(0.0), _C.c_double(0.0)
    ctx.check(lib().tt_probe_lds(ctx.handle, 1 if mfma else 0, _C.byref(b), _C.byref(t)))
    return b.value, t.value


def tt_probe_lds_load(ctx, buf, resident=True):
    """Direct-to-LDS global loads per clock per CU (bytes), from L2-resident
    windows or streaming from HBM, over a device tensor."""
    out = _C.c_double(0.0)
    nbytes = buf.numel() * buf.element_size()
    ctx.check(lib().tt_probe_lds_load(ctx.handle, _ptr(buf), nbytes, 1 if resident else 0,
                                      _C.byref(out)))
    return out.value


ISSUE_PROBES = ["fma_1wave", "fma_2waves", "exp_1wave", "exp_2waves", "mfma_1wave", "mfma_2waves",
                "mfma_beside_fma", "mfma_beside_exp"]


def tt_probe_issue(ctx, which):
    """Clocks per instruction of the two waves of a SIMD (see ISSUE_PROBES for
    `which`); 0 for an idle second wave."""
    a, b = _C.c_double(0.0), _C.c_double(0.0)
    ctx.check(lib().tt_probe_issue(ctx.handle, which, _C.byref(a), _C.byref(b)))
    return a.value, b.value
