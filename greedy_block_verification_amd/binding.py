"""ctypes binding of libsv.so (include/sv.h): argument marshalling only.

Every function here has the name of the C entry point it calls and converts
Python/torch arguments to plain pointers and sizes.  No step of the forward
runs in Python.  ``lib()`` raises if the HIP library has not been built, and
there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsv.so")

SV_OK, SV_EINVAL, SV_ESTATE, SV_ENOSPACE, SV_EDEVICE, SV_EUNSUPPORTED, SV_ESCRATCH = 0, -1, -2, -3, -4, -5, -6


class SvError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {sv_status_str(status)} ({status})")
        self.status = status


class sv_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ff", C.c_int32),
                ("vocab", C.c_int32), ("act", C.c_int32), ("weight_fmt", C.c_int32), ("tied", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float), ("page_size", C.c_int32),
                ("max_ctx", C.c_int32), ("max_k", C.c_int32), ("max_prefill_rows", C.c_int32)]


class sv_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("wqkv", "wqkv_scales", "wo", "wo_scales", "wgu", "wgu_scales",
                                           "wd", "wd_scales", "g_attn", "g_mlp")]


class sv_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("lm_head", C.c_void_p), ("g_final", C.c_void_p),
                ("layers", C.POINTER(sv_layer_weights))]


class sv_buffers(C.Structure):
    _fields_ = [("kv_pool", C.c_void_p), ("kv_pool_bytes", C.c_int64), ("page_table", C.c_void_p),
                ("n_pages", C.c_int32), ("workspace", C.c_void_p), ("workspace_bytes", C.c_int64)]


_LIB = None

# name -> (restype, argtypes); mirrors include/sv.h
SIGNATURES = {
    "sv_query_sizes": (C.c_int, [C.POINTER(sv_config), C.POINTER(C.c_int64), C.POINTER(C.c_int64)]),
    "sv_packed_linear_bytes": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int64),
                                         C.POINTER(C.c_int64)]),
    "sv_pack_linear": (C.c_int, [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                 C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "sv_create": (C.c_int, [C.POINTER(sv_config), C.POINTER(sv_weights), C.POINTER(sv_buffers), C.c_void_p,
                            C.POINTER(C.c_void_p)]),
    "sv_destroy": (None, [C.c_void_p]),
    "sv_prefill": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32, C.POINTER(C.c_int32)]),
    "sv_decode_step": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32)]),
    "sv_verify": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.c_int32, C.POINTER(C.c_int32),
                            C.POINTER(C.c_int32)]),
    "sv_verify_noalloc": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.c_int32, C.POINTER(C.c_int32),
                                    C.POINTER(C.c_int32)]),
    "sv_verify_batch": (C.c_int, [C.POINTER(C.c_void_p), C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                  C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "sv_kv_truncate": (C.c_int, [C.c_void_p, C.c_int32]),
    "sv_topk": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_float)]),
    "sv_selected_logits": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.c_int32,
                                     C.POINTER(C.c_float)]),
    "sv_clone_state": (C.c_int, [C.c_void_p, C.c_void_p]),
    "sv_kv_len": (C.c_int32, [C.c_void_p]),
    "sv_next_id": (C.c_int32, [C.c_void_p]),
    "sv_set_debug": (C.c_int, [C.c_void_p, C.c_int32]),
    "sv_get_logits": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32]),
    "sv_last_argmax": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "sv_history": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32]),
    "sv_restore": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32)]),
    "sv_set_profile": (C.c_int, [C.c_void_p, C.c_int32]),
    "sv_profile_read": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
    "sv_profile_reset": (C.c_int, [C.c_void_p]),
    "sv_status_str": (C.c_char_p, [C.c_int]),
}


def lib():
    """Load libsv.so (built in-tree by ``build.py``); raise if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python greedy_block_verification_amd/build.py` (there is no fallback)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _LIB = L
    return _LIB


def _check(status: int, where: str):
    if status != SV_OK:
        raise SvError(status, where)


def sv_status_str(status: int) -> str:
    return lib().sv_status_str(status).decode()


def _i32_array(vals):
    vals = [int(v) for v in vals]
    return (C.c_int32 * max(1, len(vals)))(*vals)


def make_config(cfg, max_prefill_rows: int = 0) -> sv_config:
    """sv_config from a ``seeded_inputs.ModelConfig`` (max_prefill_rows: rows of
    one row-tiled prefill forward, 0 for 64-row forwards only)."""
    return sv_config(cfg.n_layers, cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_ff,
                     cfg.vocab, 0 if cfg.act == "swiglu" else 1, 0 if cfg.weight_fmt == "bf16" else 1,
                     1 if cfg.tied else 0, cfg.rms_eps, cfg.rope_theta, cfg.page_size, cfg.max_ctx, cfg.max_k,
                     int(max_prefill_rows))


def sv_query_sizes(cfg: sv_config):
    kv, ws = C.c_int64(), C.c_int64()
    _check(lib().sv_query_sizes(C.byref(cfg), C.byref(kv), C.byref(ws)), "sv_query_sizes")
    return kv.value, ws.value


def sv_packed_linear_bytes(fmt: int, n: int, k: int):
    b, s = C.c_int64(), C.c_int64()
    _check(lib().sv_packed_linear_bytes(fmt, n, k, C.byref(b), C.byref(s)), "sv_packed_linear_bytes")
    return b.value, s.value


def sv_pack_linear(fmt, layout, src0, src0_scales, src1, src1_scales, n, k, head_dim, dst, dst_scales, stream):
    _check(lib().sv_pack_linear(fmt, layout, src0, src0_scales, src1, src1_scales, n, k, head_dim, dst, dst_scales,
                                stream), "sv_pack_linear")


def sv_create(cfg: sv_config, weights: sv_weights, buffers: sv_buffers, stream) -> int:
    h = C.c_void_p()
    _check(lib().sv_create(C.byref(cfg), C.byref(weights), C.byref(buffers), stream, C.byref(h)), "sv_create")
    return h.value


def sv_destroy(ctx):
    lib().sv_destroy(ctx)


def sv_prefill(ctx, ids) -> int:
    nx = C.c_int32()
    _check(lib().sv_prefill(ctx, _i32_array(ids), len(ids), C.byref(nx)), "sv_prefill")
    return nx.value


def sv_decode_step(ctx, token: int) -> int:
    nx = C.c_int32()
    _check(lib().sv_decode_step(ctx, int(token), C.byref(nx)), "sv_decode_step")
    return nx.value


def sv_verify(ctx, prefix_len: int, draft_ids):
    n, nx = C.c_int32(), C.c_int32()
    _check(lib().sv_verify(ctx, int(prefix_len), _i32_array(draft_ids), len(draft_ids), C.byref(n), C.byref(nx)),
           "sv_verify")
    return n.value, nx.value


def sv_verify_noalloc(ctx, prefix_len: int, draft_ids):
    n, nx = C.c_int32(), C.c_int32()
    _check(lib().sv_verify_noalloc(ctx, int(prefix_len), _i32_array(draft_ids), len(draft_ids), C.byref(n),
                                   C.byref(nx)), "sv_verify_noalloc")
    return n.value, nx.value


def sv_verify_batch(ctxs, prefix_lens, drafts):
    """drafts: one list of draft ids per context; returns [(n_accepted, next_id)]."""
    n = len(ctxs)
    arr = (C.c_void_p * n)(*ctxs)
    flat = [int(t) for d in drafts for t in d]
    na, nx = (C.c_int32 * n)(), (C.c_int32 * n)()
    _check(lib().sv_verify_batch(arr, n, _i32_array(prefix_lens), _i32_array([len(d) for d in drafts]),
                                 _i32_array(flat), na, nx), "sv_verify_batch")
    return [(na[i], nx[i]) for i in range(n)]


def sv_topk(ctx, row: int, k: int):
    """[(id, logit)] of the k largest logits of a row of the last forward."""
    ids, vals = (C.c_int32 * k)(), (C.c_float * k)()
    _check(lib().sv_topk(ctx, int(row), int(k), ids, vals), "sv_topk")
    return [(ids[i], vals[i]) for i in range(k)]


def sv_selected_logits(ctx, row: int, ids):
    n = len(ids)
    vals = (C.c_float * max(1, n))()
    _check(lib().sv_selected_logits(ctx, int(row), _i32_array(ids), n, vals), "sv_selected_logits")
    return [vals[i] for i in range(n)]


def sv_clone_state(dst, src):
    _check(lib().sv_clone_state(dst, src), "sv_clone_state")


def sv_kv_truncate(ctx, new_len: int):
    _check(lib().sv_kv_truncate(ctx, int(new_len)), "sv_kv_truncate")


def sv_kv_len(ctx) -> int:
    return lib().sv_kv_len(ctx)


def sv_next_id(ctx) -> int:
    return lib().sv_next_id(ctx)


def sv_set_debug(ctx, store_logits: int):
    _check(lib().sv_set_debug(ctx, int(store_logits)), "sv_set_debug")


def sv_get_logits(ctx, row: int, vocab: int):
    import numpy as np
    out = np.empty(vocab, dtype=np.float32)
    _check(lib().sv_get_logits(ctx, int(row), out.ctypes.data, vocab), "sv_get_logits")
    return out


def sv_last_argmax(ctx, max_rows: int = 64):
    buf = (C.c_int32 * max(64, int(max_rows)))()
    m = C.c_int32()
    _check(lib().sv_last_argmax(ctx, buf, C.byref(m)), "sv_last_argmax")
    return list(buf[:m.value])


def sv_set_profile(ctx, mask: int):
    _check(lib().sv_set_profile(ctx, int(mask)), "sv_set_profile")


def sv_profile_read(ctx, role: int):
    ms, n = C.c_double(), C.c_int64()
    _check(lib().sv_profile_read(ctx, int(role), C.byref(ms), C.byref(n)), "sv_profile_read")
    return ms.value, n.value


def sv_profile_reset(ctx):
    _check(lib().sv_profile_reset(ctx), "sv_profile_reset")


def sv_history(ctx, n: int):
    buf = (C.c_int32 * max(1, n))()
    _check(lib().sv_history(ctx, buf, int(n)), "sv_history")
    return list(buf[:n])


def sv_restore(ctx, kv_len: int, greedy_hist):
    _check(lib().sv_restore(ctx, int(kv_len), _i32_array(greedy_hist)), "sv_restore")
