"""Device set-up of a KVSwap workload from the seeded generators.

Builds, for a ``lsa_inputs.KVSwapWorkload``: the low-rank factors U, S, V of
every segment (segment s = (layer * groups + group) * batch + b), the cold
K/V store of every (group, sequence) -- shared by all layers --, one
``lsa.Pool`` per (layer, group) whose slot rows are laid out back to back,
the per-step group queries and the output buffers of ``lsa.kvswap_step``.
The f16 tensors are uploaded as uint8 codes and expanded through the code
table on the device (an exact table lookup).  No arithmetic of the method
happens here.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

import lsa_inputs as L

from . import lsa


def _table(n_points: int, offset: int, dev) -> torch.Tensor:
    t = torch.from_numpy(L.code_table_f16(n_points, offset).view(np.int16)).to(dev)
    return t.view(torch.float16)


class DeviceKVSwap:
    def __init__(self, wl: L.KVSwapWorkload, device: int = 0, ctx: Optional[lsa.Ctx] = None, log=None):
        self.wl = wl
        self.dev = torch.device(f"cuda:{device}")
        self.ctx = ctx if ctx is not None else lsa.Ctx(device)
        say = log or (lambda *_: None)
        B, G, T, r, C = wl.batch, wl.groups, wl.ctx, wl.rank, wl.C
        n_seg, P, S = wl.n_seg, wl.n_pools, wl.slots
        dev = self.dev
        lut_u = _table(L.U_POINTS, L.U_OFFSET, dev)
        lut_kv = _table(L.KV_POINTS, L.KV_OFFSET, dev)
        self.U = torch.empty((n_seg, T, r), dtype=torch.float16, device=dev)
        self.V = torch.empty((n_seg, C, r), dtype=torch.float16, device=dev)
        S_host = np.empty((n_seg, r), np.float32)
        per_layer = G * B
        for l in range(wl.layers):
            cu = np.empty((per_layer, T, r), np.uint8)
            cv = np.empty((per_layer, C, r), np.uint8)
            for g in range(G):
                for b in range(B):
                    cu[g * B + b] = L.lowrank_U_codes(wl, l, g, b)
                    cv[g * B + b] = L.lowrank_V_codes(wl, l, g, b)
                    S_host[wl.seg(l, g, b)] = L.lowrank_S(wl, l, g, b)
            s0 = l * per_layer
            self.U[s0:s0 + per_layer] = lut_u[torch.from_numpy(cu).to(dev).int()]
            self.V[s0:s0 + per_layer] = lut_u[torch.from_numpy(cv).to(dev).int()]
        self.S = torch.from_numpy(S_host).to(dev)
        say(f"factors: U {tuple(self.U.shape)} f16, V {tuple(self.V.shape)} f16")
        # cold K/V per (group, sequence), shared by all layers
        self.cold = torch.empty((G, B, T, 2 * C), dtype=torch.float16, device=dev)
        for g in range(G):
            for b in range(B):
                self.cold[g, b] = lut_kv[torch.from_numpy(L.kvswap_cold_codes(wl, g, b)).to(dev).int()]
        say(f"cold K/V {tuple(self.cold.shape)} f16 ({self.cold.numel() * 2 / 2**30:.2f} GiB)")
        # slot rows of every pool back to back: [P][B][S][2C]
        self.kv = torch.zeros((P, B, S, 2 * C), dtype=torch.float16, device=dev)
        self.pools: List[lsa.Pool] = []
        row_bytes = 2 * C * 2
        for p in range(P):
            g = p % G
            pool = lsa.Pool(T, 1, self.kv[p], 0, S, wl.k, kv_dim=2 * C, batch=B, cold="hbm",
                            kv_stride_b=S * 2 * C, cold_buf=self.cold[g], cold_stride_b=T * row_bytes)
            for b in range(B):
                pool.mark_stored(b, 0, T)
            if wl.recency_w < 100 or wl.high_water < 100:
                pool.set_replacement(wl.recency_w, wl.high_water)
            self.pools.append(pool)
        if not self.pools[0].swap:
            # slots for every position: the pools never swap and read row t at slot t,
            # so the rows are resident from the start
            for p in range(P):
                self.kv[p, :, :T] = self.cold[p % G]
        torch.cuda.synchronize()
        say(f"{P} pools of {S} slots x batch {B}, swap={self.pools[0].swap}")
        self.scores = torch.zeros((n_seg, T), dtype=torch.float32, device=dev)
        self.sel = torch.zeros((n_seg, wl.k), dtype=torch.int32, device=dev)
        self.count = torch.zeros((n_seg,), dtype=torch.int32, device=dev)
        self.phys = torch.zeros((n_seg, wl.k), dtype=torch.int32, device=dev)
        self.n_rows = torch.zeros((n_seg,), dtype=torch.int32, device=dev)
        self.out = torch.zeros((n_seg, wl.group_heads, wl.head_dim), dtype=torch.float32, device=dev)
        self.q = None
        self.q_np = None

    def make_steps(self, steps: int) -> None:
        """Draw the group queries of steps 0..steps-1 ([steps][n_seg][C]) and upload them."""
        wl = self.wl
        q = np.empty((steps, wl.n_seg, wl.C), np.float32)
        for l in range(wl.layers):
            for g in range(wl.groups):
                for b in range(wl.batch):
                    q[:, wl.seg(l, g, b)] = L.kvswap_query_steps(wl, l, g, b, steps)
        self.q_np = q
        self.q = torch.from_numpy(q).to(self.dev)

    def step(self, t: int, stream=None, fused: bool = False) -> None:
        """Step t; fused: no scores buffer, so score and top-k run as one launch."""
        wl = self.wl
        lsa.kvswap_step(self.ctx, U=self.U, S=self.S, V=self.V, q=self.q[t], pools=self.pools, k=wl.k,
                        heads=wl.group_heads, head_dim=wl.head_dim, scores=None if fused else self.scores,
                        sel=self.sel,
                        count=self.count, phys=self.phys, n_rows=self.n_rows, out=self.out, scale=wl.scale,
                        stream=stream)

    def reset_pools(self) -> None:
        for p in self.pools:
            p.reset()
        torch.cuda.synchronize()

    def host_inputs(self, seg: int, t: int):
        """The oracle's inputs of one segment at step t (f16 codes for U, V and the cold rows)."""
        wl = self.wl
        b = seg % wl.batch
        g = (seg // wl.batch) % wl.groups
        l = seg // (wl.batch * wl.groups)
        U = L.f32_to_f16_bits(L.lowrank_U(wl, l, g, b))
        V = L.f32_to_f16_bits(L.lowrank_V(wl, l, g, b))
        S = L.lowrank_S(wl, l, g, b)
        cold = L.f32_to_f16_bits(L.kvswap_cold(wl, g, b))
        return U, S, V, self.q_np[t, seg], cold
