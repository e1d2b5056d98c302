"""A second fp64 formulation of the model on torch-CPU library routines.

Used only to pin the oracle: RMSNorm is ``F.rms_norm``, attention is
``F.scaled_dot_product_attention(is_causal=True)`` with KV heads expanded by
``repeat_interleave``, the gates are ``F.silu`` / ``F.gelu(approximate='tanh')``
and RoPE is written as a complex rotation of the pairs (u_i, u_{i+dh/2}).
"""
import torch
import torch.nn.functional as F


def _t(bits_or_arr):
    import numpy as np
    from seeded_inputs.weights import f32_from_bf16_bits
    a = np.asarray(bits_or_arr)
    if a.dtype == np.uint16:
        a = f32_from_bf16_bits(a)
    return torch.from_numpy(a.astype(np.float64))


def linear_f64(w, layer, name):
    cfg = w.cfg
    L = w.layers[layer]
    if cfg.weight_fmt == "int4":
        q = torch.from_numpy(L[name].astype("float64"))
        s = _t(L[name + "_s"])
        return q * torch.repeat_interleave(s, 64, dim=1)
    return _t(L[name])


def rope_complex(u, pos, theta):
    # u: [T, H, dh] float64; pairs (i, i + dh/2) rotated by pos * theta^(-2i/dh)
    T, H, dh = u.shape
    half = dh // 2
    freqs = torch.pow(torch.tensor(theta, dtype=torch.float64),
                      -torch.arange(0, dh, 2, dtype=torch.float64) / dh)
    ang = torch.outer(pos.to(torch.float64), freqs)
    z = torch.complex(u[..., :half], u[..., half:]) * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1)


def forward(w, tokens):
    cfg = w.cfg
    ids = torch.tensor(list(tokens), dtype=torch.long)
    T = len(ids)
    E = _t(w.embed)
    x = F.embedding(ids, E)
    pos = torch.arange(T)
    act = F.silu if cfg.act == "swiglu" else (lambda z: F.gelu(z, approximate="tanh"))
    for l in range(cfg.n_layers):
        g_a = _t(w.layers[l]["g_attn"])
        g_m = _t(w.layers[l]["g_mlp"])
        h = F.rms_norm(x, (cfg.d_model,), weight=g_a, eps=cfg.rms_eps)
        q = F.linear(h, linear_f64(w, l, "wq")).view(T, cfg.n_q_heads, cfg.head_dim)
        k = F.linear(h, linear_f64(w, l, "wk")).view(T, cfg.n_kv_heads, cfg.head_dim)
        v = F.linear(h, linear_f64(w, l, "wv")).view(T, cfg.n_kv_heads, cfg.head_dim)
        q = rope_complex(q, pos, cfg.rope_theta)
        k = rope_complex(k, pos, cfg.rope_theta)
        k = torch.repeat_interleave(k, cfg.group, dim=1)
        v = torch.repeat_interleave(v, cfg.group, dim=1)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1),
                                           v.transpose(0, 1), is_causal=True)
        x = x + F.linear(o.transpose(0, 1).reshape(T, -1), linear_f64(w, l, "wo"))
        h = F.rms_norm(x, (cfg.d_model,), weight=g_m, eps=cfg.rms_eps)
        a = act(F.linear(h, linear_f64(w, l, "wg"))) * F.linear(h, linear_f64(w, l, "wu"))
        x = x + F.linear(a, linear_f64(w, l, "wd"))
    h = F.rms_norm(x, (cfg.d_model,), weight=_t(w.g_final), eps=cfg.rms_eps)
    return F.linear(h, E).numpy()
