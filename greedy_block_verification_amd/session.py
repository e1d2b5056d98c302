"""Device model and one-sequence session over libsv.so.

PyTorch provides device memory and the stream; every computation (weight
packing included) runs in the HIP library.  ``DeviceModel`` uploads a
``seeded_inputs.ModelWeights`` and packs it with ``sv_pack_linear``;
``Session`` owns one context (one sequence) with its KV pool, page table and
workspace.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import binding as B


def _dev(arr: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceModel:
    """Packed device weights of one model (shared by any number of sessions)."""

    def __init__(self, weights, device="cuda:0", share_layers_with=None):
        import torch.cuda
        if not torch.cuda.is_available():
            raise RuntimeError("DeviceModel needs a ROCm GPU")
        B.lib()
        self.cfg = weights.cfg
        self.device = torch.device(device)
        self.stream = torch.cuda.current_stream(self.device)
        self.keep = []                      # device tensors the contexts point into
        cfg = self.cfg
        fmt = 0 if cfg.weight_fmt == "bf16" else 1
        self.fmt = fmt
        self.embed = self._pack(0, 0, weights.embed, None)[0]
        self.g_final = self._keep(_dev(weights.g_final, self.device))
        self.layer_structs = (B.sv_layer_weights * cfg.n_layers)()
        if share_layers_with is not None:
            # same layer weights (device memory shared), own embedding / LM head
            self.keep.append(share_layers_with)
            for l in range(cfg.n_layers):
                self.layer_structs[l] = share_layers_with.layer_structs[l]
        for l, L in enumerate(weights.layers if share_layers_with is None else []):
            qkv = np.concatenate([L["wq"], L["wk"], L["wv"]], axis=0)
            qkv_s = np.concatenate([L["wq_s"], L["wk_s"], L["wv_s"]], axis=0) if fmt else None
            wqkv, wqkv_s = self._pack(fmt, 2, qkv, qkv_s)
            wo, wo_s = self._pack(fmt, 0, L["wo"], L.get("wo_s"))
            wgu, wgu_s = self._pack(fmt, 1, L["wg"], L.get("wg_s"), L["wu"], L.get("wu_s"))
            wd, wd_s = self._pack(fmt, 0, L["wd"], L.get("wd_s"))
            ga = self._keep(_dev(L["g_attn"], self.device))
            gm = self._keep(_dev(L["g_mlp"], self.device))
            s = self.layer_structs[l]
            s.wqkv, s.wo, s.wgu, s.wd = wqkv, wo, wgu, wd
            s.wqkv_scales, s.wo_scales, s.wgu_scales, s.wd_scales = wqkv_s, wo_s, wgu_s, wd_s
            s.g_attn, s.g_mlp = ga, gm
        torch.cuda.synchronize(self.device)
        self.weights = B.sv_weights(self.embed, self.embed, self.g_final, self.layer_structs)
        self.config = B.make_config(cfg)

    def _keep(self, t: torch.Tensor) -> int:
        self.keep.append(t)
        return t.data_ptr()

    def _pack(self, fmt, layout, w0, s0, w1=None, s1=None):
        n, k = w0.shape
        nb, sb = B.sv_packed_linear_bytes(fmt, n * (2 if w1 is not None else 1), k)
        dst = torch.empty(nb, dtype=torch.uint8, device=self.device)
        dst_s = torch.empty(max(sb, 1), dtype=torch.uint8, device=self.device) if fmt else None
        t0 = _dev(w0, self.device)
        t1 = _dev(w1, self.device) if w1 is not None else None
        ts0 = _dev(s0, self.device) if fmt else None
        ts1 = _dev(s1, self.device) if (fmt and w1 is not None) else None
        B.sv_pack_linear(fmt, layout, t0.data_ptr(), ts0.data_ptr() if ts0 is not None else None,
                         t1.data_ptr() if t1 is not None else None, ts1.data_ptr() if ts1 is not None else None,
                         n, k, self.cfg.head_dim, dst.data_ptr(), dst_s.data_ptr() if dst_s is not None else None,
                         self.stream.cuda_stream)
        torch.cuda.synchronize(self.device)
        del t0, t1, ts0, ts1
        return self._keep(dst), (self._keep(dst_s) if dst_s is not None else None)


class Session:
    """One sequence: a context with its own KV pool, page table and workspace.

    ``page_perm`` optionally scatters logical pages over physical pages (a
    permutation of range(n_pages)), to exercise the page table.
    ``poison`` fills the KV pool with NaN bit patterns first, so a read past
    the committed length would reach the logits.
    """

    def __init__(self, model: DeviceModel, page_perm=None, poison: bool = False, cfg=None, prefill_rows: int = 0):
        self.m = model
        cfg = cfg or model.cfg
        self.cfg = cfg
        self.prefill_rows = int(prefill_rows)
        config = B.make_config(cfg, self.prefill_rows)
        self.config = config
        kv_bytes, ws_bytes = B.sv_query_sizes(config)
        n_pages = cfg.max_ctx // cfg.page_size
        dev = model.device
        self.kv = torch.empty(kv_bytes // 2, dtype=torch.int16, device=dev)
        if poison:
            self.kv.fill_(0x7FC1)            # fp16 NaN pattern
        else:
            self.kv.zero_()
        perm = np.arange(n_pages, dtype=np.int32) if page_perm is None else np.asarray(page_perm, dtype=np.int32)
        self.page_table = torch.from_numpy(perm.copy()).to(dev)
        self.ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize(dev)
        self.buffers = B.sv_buffers(self.kv.data_ptr(), kv_bytes, self.page_table.data_ptr(), n_pages,
                                    self.ws.data_ptr(), ws_bytes)
        self.ctx = B.sv_create(config, model.weights, self.buffers, model.stream.cuda_stream)

    def close(self):
        if self.ctx:
            B.sv_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # thin pass-throughs
    def prefill(self, ids) -> int:
        return B.sv_prefill(self.ctx, ids)

    def decode_step(self, token: int) -> int:
        return B.sv_decode_step(self.ctx, token)

    def verify(self, drafts):
        return B.sv_verify(self.ctx, B.sv_kv_len(self.ctx), drafts)

    def truncate(self, new_len: int):
        B.sv_kv_truncate(self.ctx, new_len)

    @property
    def kv_len(self) -> int:
        return B.sv_kv_len(self.ctx)

    @property
    def next_id(self) -> int:
        return B.sv_next_id(self.ctx)

    def set_debug(self, on: bool):
        B.sv_set_debug(self.ctx, 1 if on else 0)

    def logits(self, row: int) -> np.ndarray:
        return B.sv_get_logits(self.ctx, row, self.cfg.vocab)

    def last_argmax(self):
        return B.sv_last_argmax(self.ctx, self.prefill_rows)

    def history(self, n=None):
        return B.sv_history(self.ctx, self.kv_len if n is None else n)

    def snapshot(self):
        """(KV pool copy, greedy history): everything a restore needs."""
        torch.cuda.synchronize(self.kv.device)
        return self.kv.clone(), self.history()

    def restore(self, snap):
        kv, hist = snap
        self.kv.copy_(kv)
        torch.cuda.synchronize(self.kv.device)
        B.sv_restore(self.ctx, len(hist), hist)

    def kv_positions(self, n_positions: int, start: int = 0) -> np.ndarray:
        """Host copy of the K/V bits of positions [start, n): int16 [n - start, L, 2, n_kv, dh]."""
        cfg = self.cfg
        n_pages = cfg.max_ctx // cfg.page_size
        ps, dh = cfg.page_size, cfg.head_dim
        pool = self.kv.view(cfg.n_layers, n_pages, 2, cfg.n_kv_heads, ps * dh)
        pt = self.page_table.cpu().numpy()
        pos = np.arange(start, n_positions)
        pages = pt[pos // ps].astype(np.int64)
        upages, inv = np.unique(pages, return_inverse=True)
        sub = pool[:, torch.from_numpy(upages).to(self.kv.device)].cpu().numpy()   # [L, u, 2, nkv, 16*dh]
        L, u = sub.shape[0], sub.shape[1]
        k = sub[:, :, 0].reshape(L, u, cfg.n_kv_heads, ps, dh)
        v = sub[:, :, 1].reshape(L, u, cfg.n_kv_heads, dh, ps).transpose(0, 1, 2, 4, 3)   # V is [dh][slot] in a page
        kv = np.stack([k, v], axis=2)                                              # [L, u, 2, nkv, 16, dh]
        return kv[:, inv, :, :, pos % ps, :]                                       # [n, L, 2, nkv, dh]
