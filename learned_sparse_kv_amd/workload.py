"""Device set-up of a decode-step workload from the seeded generators.

Builds, for a ``lsa_inputs.Workload``: the source layer's indexer keys in HBM,
one ``lsa.Pool`` per sparse layer (window rows in the KV buffer, every
compressed row stored in the cold pool -- pinned host memory is filled in
place), the per-step indexer and attention queries, and the output buffers of
``lsa.decode_step``.  No arithmetic of the method happens here.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

import lsa_inputs as L

from . import lsa


def to_device(x, dtype: str, dev):
    """Upload values already encoded for `dtype` (f32 array, bf16/f16 16-bit codes
    or fp8 E4M3 byte codes); for the MX dtypes an MXKeys becomes (codes, scales)
    tensors (float4_e2m1fn_x2 or int8 codes, float8_e8m0fnu scales)."""
    if dtype in L.MX_DTYPES:
        codes = torch.from_numpy(np.ascontiguousarray(x.codes)).to(dev)
        if dtype == "mxfp4":
            codes = codes.view(torch.float4_e2m1fn_x2)
        scales = torch.from_numpy(np.ascontiguousarray(x.scales, dtype=np.uint8)).to(dev).view(torch.float8_e8m0fnu)
        return codes, scales
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(dev).view(torch.float8_e4m3fn)
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "fp8": torch.float8_e4m3fn}[dtype]


class DeviceWorkload:
    """stored: optional per-layer count of leading entries stored at set-up (the
    rest are stored later with store(); default all).  n_valid: optional valid
    source entries per sequence, passed to every step (default all)."""

    def __init__(self, wl: L.Workload, device: int = 0, keep_host: bool = False, ctx: Optional[lsa.Ctx] = None,
                 log=None, stored: Optional[List[int]] = None):
        self.wl = wl
        self.dev = torch.device(f"cuda:{device}")
        self.ctx = ctx if ctx is not None else lsa.Ctx(device)
        self.keep_host = keep_host
        say = log or (lambda *_: None)
        B, D, W = wl.batch, wl.kv_dim, wl.window
        keys_np = [L.indexer_keys(wl, b) for b in range(B)]
        self.keys = to_device(L.stack_keys(keys_np, wl.key_dtype), wl.key_dtype, self.dev)
        self.key_scales = None
        if wl.key_dtype in L.MX_DTYPES:
            self.keys, self.key_scales = self.keys
        self.keys_np = keys_np if keep_host else None
        say(f"keys {tuple(self.keys.shape)} {wl.key_dtype}")
        self.pools: List[lsa.Pool] = []
        self.kv: List[torch.Tensor] = []
        self.windows: List[List[np.ndarray]] = []
        self.stores: List[List[np.ndarray]] = []
        np_row = np.float32 if wl.kv_dtype == "f32" else np.uint16
        for l in range(wl.n_layers):
            rows = lsa.Pool.rows_needed(wl.ctx, wl.layer_ratios[l], W, wl.gpu_chunks)
            kv = torch.zeros((B, rows, D), dtype=torch_dtype(wl.kv_dtype), device=self.dev)
            pool = lsa.Pool(wl.ctx, wl.layer_ratios[l], kv, W, wl.gpu_chunks, wl.k, D, B, cold=wl.cold)
            if pool.swap and (wl.recency_w < 100 or wl.high_water < 100):
                pool.set_replacement(wl.recency_w if wl.layer_ratios[l] == wl.src_ratio else 100, wl.high_water)
            wins, stores = [], []
            for b in range(B):
                win = L.encode(L.window_rows(wl, l, b), wl.kv_dtype)
                kv[b, :W] = to_device(win, wl.kv_dtype, self.dev)
                host = pool.host_rows(b, np_row)
                n0 = pool.cap if stored is None else int(stored[l])
                if host is not None and wl.kv_dtype == "f32":
                    L.cold_rows(wl, l, b, out=host)
                    pool.mark_stored(b, 0, n0)
                    store = host
                elif host is not None:
                    host[:] = L.encode(L.cold_rows(wl, l, b), wl.kv_dtype)
                    pool.mark_stored(b, 0, n0)
                    store = host
                else:
                    store = L.encode(L.cold_rows(wl, l, b), wl.kv_dtype)
                    pool.store(b, 0, store[:n0])
                wins.append(win)
                stores.append(store if keep_host else None)
            self.pools.append(pool)
            self.kv.append(kv)
            self.windows.append(wins)
            self.stores.append(stores)
            say(f"layer {l}: ratio {wl.layer_ratios[l]} cap {pool.cap} swap {pool.swap} cold {wl.cold}")
        torch.cuda.synchronize()
        nL, k = wl.n_layers, wl.k
        self.scores = torch.zeros((B, wl.n_src), dtype=torch.float32, device=self.dev)
        self.sel = torch.zeros((B, k), dtype=torch.int32, device=self.dev)
        self.count = torch.zeros((B,), dtype=torch.int32, device=self.dev)
        self.out = torch.zeros((nL, B, wl.hq, D), dtype=torch.float32, device=self.dev)
        self.phys = torch.zeros((nL, B, W + k), dtype=torch.int32, device=self.dev)
        self.n_rows = torch.zeros((nL, B), dtype=torch.int32, device=self.dev)
        self.q_idx = self.w_idx = self.q_attn = None
        self.q_idx_np = self.w_idx_np = self.q_attn_np = None
        self.n_valid = None

    def store(self, l: int, b: int, first: int, rows: np.ndarray) -> None:
        """Store rows (encoded in the row dtype) into entries first.. of layer l,
        sequence b (lsa_pool_store), keeping the host copy in step."""
        self.pools[l].store(b, first, np.ascontiguousarray(rows))
        if self.keep_host and self.stores[l][b] is not None and self.pools[l].host_rows(b) is None:
            self.stores[l][b][first:first + rows.shape[0]] = rows

    def make_steps(self, steps: int) -> None:
        """Draw the indexer and attention queries of `steps` steps and upload them."""
        wl = self.wl
        B, nL = wl.batch, wl.n_layers
        qs, ws = [], []
        for b in range(B):
            q, w = L.indexer_query_steps(wl, b, steps)
            qs.append(q)
            ws.append(w)
        self.q_idx_np = np.stack(qs, axis=1)          # [steps][B][n_idx][H][dk]
        self.w_idx_np = np.stack(ws, axis=1)          # [steps][B][n_idx][H]
        self.q_attn_np = np.stack([np.stack([np.stack([L.attn_query(wl, l, b, t) for b in range(B)])
                                             for l in range(nL)]) for t in range(steps)])
        self.q_idx = torch.from_numpy(self.q_idx_np).to(self.dev)
        self.w_idx = torch.from_numpy(self.w_idx_np).to(self.dev)
        self.q_attn = torch.from_numpy(self.q_attn_np).to(self.dev)

    def _step_args(self, t: int):
        wl = self.wl
        return dict(keys=self.keys, q_idx=self.q_idx[t], w_idx=self.w_idx[t], pools=self.pools,
                    q_attn=self.q_attn[t], out=self.out, scores=self.scores, sel=self.sel, count=self.count,
                    k=wl.k, src_ratio=wl.src_ratio, scale=wl.scale, ensemble=wl.ensemble, mode=wl.mode,
                    tau=wl.tau if wl.tau is not None else 0.5, phys=self.phys, n_rows=self.n_rows,
                    key_scales=self.key_scales, n_valid=self.n_valid)

    def step(self, t: int, stream=None) -> None:
        lsa.decode_step(self.ctx, stream=stream, **self._step_args(t))

    def attend(self, t: int, stream=None) -> None:
        """Step t of the window the last prediction serves (lsa_decode_attend)."""
        lsa.decode_attend(self.ctx, stream=stream, **self._step_args(t))

    # ---- lookahead schedule: step t attends with the rows staged during step
    # t-1 (or by prime) and predicts step t+1 from q_idx[t+1]
    def _la_buffers(self):
        if getattr(self, "phys2", None) is None:
            wl = self.wl
            self.phys2 = torch.zeros((2, wl.n_layers, wl.batch, wl.window + wl.k), dtype=torch.int32, device=self.dev)
            self.n_rows2 = torch.zeros((2, wl.n_layers, wl.batch), dtype=torch.int32, device=self.dev)

    def _la_args(self, t_idx: int, t_attn: int):
        wl = self.wl
        self._la_buffers()
        return dict(keys=self.keys, q_idx=self.q_idx[t_idx], w_idx=self.w_idx[t_idx], pools=self.pools,
                    q_attn=self.q_attn[t_attn], out=self.out, scores=self.scores, sel=self.sel, count=self.count,
                    k=wl.k, src_ratio=wl.src_ratio, scale=wl.scale, ensemble=wl.ensemble, mode=wl.mode,
                    tau=wl.tau if wl.tau is not None else 0.5, phys=self.phys2, n_rows=self.n_rows2,
                    key_scales=self.key_scales, n_valid=self.n_valid)

    def lookahead_prime(self, t: int = 0, stream=None) -> None:
        lsa.lookahead_prime(self.ctx, stream=stream, **self._la_args(t, t))

    def lookahead_step(self, t: int, stream=None, t_next: Optional[int] = None) -> None:
        """Attend step t and stage the next prediction from the indexer query of step
        t_next (default t+1)."""
        lsa.lookahead_step(self.ctx, stream=stream, **self._la_args(t + 1 if t_next is None else t_next, t))

    def lookahead_attend(self, t: int, stream=None) -> None:
        """Attend step t over the current prediction's rows (lsa_lookahead_attend)."""
        lsa.lookahead_attend(self.ctx, stream=stream, **self._la_args(t, t))

    def prepare_lookahead(self, steps) -> None:
        """Marshal the descriptors of the listed lookahead steps once (launch with run_prepared)."""
        self.prepared = {t: lsa.PreparedStep("lsa_lookahead_step", self.ctx, **self._la_args(t + 1, t))
                         for t in steps}

    def prepare_periodic(self, steps, period: int) -> None:
        """Marshal the descriptors of the listed steps of the periodic-indexer schedule once:
        lsa_lookahead_step on the last step of each window of `period` steps (predicting
        the next step), lsa_lookahead_attend on the others (launch with run_prepared)."""
        self.prepared = {t: (lsa.PreparedStep("lsa_lookahead_step", self.ctx, **self._la_args(t + 1, t))
                             if (t + 1) % period == 0 else
                             lsa.PreparedStep("lsa_lookahead_attend", self.ctx, **self._la_args(t, t)))
                         for t in steps}

    def prepare_steps(self, steps) -> None:
        """Marshal the descriptors of the listed synchronous steps once (launch with run_prepared)."""
        self.prepared = {t: lsa.PreparedStep("lsa_decode_step", self.ctx, **self._step_args(t)) for t in steps}

    def run_prepared(self, t: int) -> None:
        self.prepared[t]()

    def capture_lookahead(self, steps) -> None:
        self.graphs = {}
        for t in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.lookahead_step(t)
            self.graphs[t] = g
        torch.cuda.synchronize()

    def capture(self, steps) -> None:
        """Capture each listed step as a HIP graph (torch.cuda.CUDAGraph around
        one lsa.decode_step).  The step enqueues only kernel launches, so the
        graph replays exactly the eager work; run one eager step first so the
        context workspace is already sized."""
        self.graphs = {}
        for t in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(t)
            self.graphs[t] = g
        torch.cuda.synchronize()

    def replay(self, t: int) -> None:
        self.graphs[t].replay()

    def reset_pools(self) -> None:
        for p in self.pools:
            p.reset()
        torch.cuda.synchronize()
