"""CPU oracle of the LSA decode hot path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``learned_sparse_kv_amd``) never imports, links or calls it, and this package
never imports the product library.  The arithmetic lives in the plain C++ file
``lsa_oracle.cpp`` (double accumulation, one entry at a time); this module only
marshals numpy arrays and chains the steps in the pages' order:
score -> select -> (per sparse layer) ratio map -> stage -> attend.

Parity pins for every function are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsa_oracle.cpp")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "liblsa_oracle.so")

DT = {"f32": 0, "bf16": 1, "f16": 2, "fp8": 3, "mxfp4": 4, "mxint8": 5}
ENS = {"max": 0, "mean": 1}
MODE = {"topk": 0, "threshold": 1}
ST_NOT_STORED = 4


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (no HIP headers, no GPU)."""
    os.makedirs(_BUILD, exist_ok=True)
    stale = not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["g++", "-std=c++17", "-O2", "-shared", "-fPIC", _SRC, "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i32, i64, u64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_double
        sig = {
            "oracle_compressed_cap": (i64, [i64, i32]),
            "oracle_pinned_bytes": (u64, [i64, P, i32, i32, i32]),
            "oracle_max_capacity": (i32, [i32, i32]),
            "oracle_swap_enabled": (i32, [i64, i32]),
            "oracle_score": (None, [P, i32, P, i64, i32, P, P, i32, i32, i32, P]),
            "oracle_project": (None, [P, i32, i32, P, P, i32, i32, i32, i32, P, P]),
            "oracle_threshold_float": (f32, [f64]),
            "oracle_select": (i32, [P, i64, i32, i32, f64, P]),
            "oracle_ratio_map": (i32, [P, i32, i32, i32, i64, P]),
            "oracle_pool_new": (P, [i64, i32, i32, i64]),
            "oracle_pool_free": (None, [P]),
            "oracle_pool_store": (None, [P, i64, i64]),
            "oracle_pool_stage": (i32, [P, P, i32, P, P, P, P, P]),
            "oracle_pool_set_replacement": (None, [P, i32, i32]),
            "oracle_pool_stats": (None, [P, P]),
            "oracle_pool_set_capacity": (None, [P, i32]),
            "oracle_pool_capacity": (i32, [P]),
            "oracle_pool_adapt": (i32, [P, f64, f64, f64, i32, i32, i32, i32]),
            "oracle_pool_state": (i32, [P, P, P]),
            "oracle_attend": (None, [P, i32, i32, P, i32, P, i32, P, i32, f32, P]),
            "oracle_lowrank_score": (None, [P, i64, i32, P, P, i32, P, P]),
            "oracle_attend_kv": (None, [P, i32, P, P, i32, i64, P, i32, f32, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(_lib, name)
            fn.restype = res
            fn.argtypes = args
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _kv(a: np.ndarray, dtype: str) -> np.ndarray:
    return _c(a, {"f32": np.float32, "fp8": np.uint8, "mxfp4": np.uint8, "mxint8": np.int8}.get(dtype, np.uint16))


# ------------------------------------------------------------------ sizing --
def compressed_cap(ctx: int, ratio: int) -> int:
    return int(lib().oracle_compressed_cap(ctx, ratio))


def pinned_bytes(ctx: int, ratios: Sequence[int], kv_dim: int, elem_bytes: int) -> int:
    r = _c(list(ratios), np.int32)
    return int(lib().oracle_pinned_bytes(ctx, _p(r), len(r), kv_dim, elem_bytes))


def max_capacity(window: int, gpu_chunks: int) -> int:
    return int(lib().oracle_max_capacity(window, gpu_chunks))


def swap_enabled(cap: int, gpu_chunks: int) -> bool:
    return bool(lib().oracle_swap_enabled(cap, gpu_chunks))


# ------------------------------------------------------------------- score --
def score(keys, key_dtype: str, q: np.ndarray, w: np.ndarray,
          ensemble: str = "max", n_valid: Optional[int] = None) -> np.ndarray:
    """keys [N][dk] (f32, 16-bit or fp8 codes; for the MX dtypes a (codes, scales)
    pair: codes [N][dk/2] (fp4) or [N][dk] (int8), E8M0 scales [N][dk/32]),
    q [n_idx][H][dk], w [n_idx][H] -> e [n_valid] f32."""
    scales = None
    if key_dtype in ("mxfp4", "mxint8"):
        keys, scales = keys
        scales = _c(scales, np.uint8)
    keys = _kv(keys, key_dtype)
    q = _c(q, np.float32)
    w = _c(w, np.float32)
    n_idx, H, dk = q.shape
    n = keys.shape[0] if n_valid is None else int(n_valid)
    e = np.zeros(n, np.float32)
    lib().oracle_score(_p(keys), DT[key_dtype], _p(scales) if scales is not None else None, n, dk, _p(q), _p(w),
                       n_idx, H, ENS[ensemble], _p(e))
    return e


# -------------------------------------------------------------- projection --
def project(hidden: np.ndarray, wq: np.ndarray, ww: np.ndarray, w_dtype: str = "f32"):
    """hidden [B][d_model] f32, wq [n_idx][H][dk][d_model] and ww [n_idx][H][d_model]
    (f32 or 16-bit codes) -> q [B][n_idx][H][dk], w [B][n_idx][H] (f32)."""
    hidden = _c(hidden, np.float32)
    wq = _kv(wq, w_dtype)
    ww = _kv(ww, w_dtype)
    B, d_model = hidden.shape
    n_idx, H, dk, d2 = wq.shape
    if d2 != d_model or ww.shape != (n_idx, H, d_model):
        raise ValueError("projection shapes do not match")
    q = np.zeros((B, n_idx, H, dk), np.float32)
    w = np.zeros((B, n_idx, H), np.float32)
    lib().oracle_project(_p(hidden), B, d_model, _p(wq), _p(ww), DT[w_dtype], n_idx, H, dk, _p(q), _p(w))
    return q, w


# ------------------------------------------------------------------ select --
def threshold_float(tau: float) -> np.float32:
    return np.float32(lib().oracle_threshold_float(float(tau)))


def select(e: np.ndarray, mode: str, k: int, tau: float = 0.5,
           n_valid: Optional[int] = None) -> np.ndarray:
    e = _c(e, np.float32)
    n = e.shape[0] if n_valid is None else int(n_valid)
    out = np.zeros(max(1, min(k, n)), np.int32)
    c = lib().oracle_select(_p(e), n, MODE[mode], k, float(tau), _p(out))
    return out[:c].copy()


def ratio_map(sel: np.ndarray, src_ratio: int, layer_ratio: int, src_valid: Optional[int] = None) -> np.ndarray:
    """Source-layer selection -> this layer's ascending complete entries (src_valid: valid
    source entries; None = unbounded)."""
    sel = _c(sel, np.int32)
    out = np.zeros(max(1, sel.size), np.int32)
    sv = (1 << 62) // max(1, src_ratio) if src_valid is None else int(src_valid)
    c = lib().oracle_ratio_map(_p(sel), sel.size, src_ratio, layer_ratio, sv, _p(out))
    return out[:c].copy()


# ------------------------------------------------------------------- stage --
class Pool:
    """One sparse layer's slot pool for one sequence (the page's LRU struct)."""

    def __init__(self, cap: int, gpu_chunks: int, window: int, row_bytes: int):
        self.cap, self.gpu_chunks, self.window = cap, gpu_chunks, window
        self._h = lib().oracle_pool_new(cap, gpu_chunks, window, row_bytes)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().oracle_pool_free(h)
            self._h = None

    def store(self, first: int, count: int) -> None:
        lib().oracle_pool_store(self._h, first, count)

    def set_replacement(self, recency_weight: int = 100, high_water: int = 100) -> None:
        """[P4] §3.2 reading: replacement order weighing recency against importance
        (percent; 100 = plain LRU), and the high-water mark (percent of the capacity)."""
        lib().oracle_pool_set_replacement(self._h, int(recency_weight), int(high_water))

    def stage(self, sel: np.ndarray, importance: Optional[np.ndarray] = None):
        """-> (status, phys [W+n], misses [(logical, slot)] in processing order);
        importance [cap] f32: the step's score of every entry (weighted pools only)."""
        sel = _c(sel, np.int32)
        n = sel.size
        phys = np.zeros(self.window + n, np.int32)
        ml = np.zeros(max(1, n), np.int32)
        ms = np.zeros(max(1, n), np.int32)
        nm = ctypes.c_int32(0)
        imp = None if importance is None else _c(importance, np.float32)
        st = lib().oracle_pool_stage(self._h, _p(sel), n, _p(imp) if imp is not None else None, _p(phys), _p(ml),
                                     _p(ms), ctypes.byref(nm))
        return int(st), phys, list(zip(ml[:nm.value].tolist(), ms[:nm.value].tolist()))

    def set_capacity(self, capacity: int) -> None:
        lib().oracle_pool_set_capacity(self._h, int(capacity))

    def capacity(self) -> int:
        return int(lib().oracle_pool_capacity(self._h))

    def adapt(self, grow_miss: float, grow_h2d: float, shrink_miss: float, step: int, min_c: int, max_c: int,
              steps: int) -> int:
        """Adaptive capacity decision over the steps since the last call; -> the new capacity."""
        return int(lib().oracle_pool_adapt(self._h, float(grow_miss), float(grow_h2d), float(shrink_miss),
                                           int(step), int(min_c), int(max_c), int(steps)))

    def stats(self) -> dict:
        out = np.zeros(4, np.uint64)
        lib().oracle_pool_stats(self._h, _p(out))
        return dict(hits=int(out[0]), misses=int(out[1]), h2d_bytes=int(out[2]), d2h_bytes=int(out[3]))

    def state(self):
        """-> (slot_logical [S], lru slot ids most- to least-recent)."""
        sl = np.zeros(self.gpu_chunks, np.int32)
        lru = np.zeros(self.gpu_chunks, np.int32)
        n = lib().oracle_pool_state(self._h, _p(sl), _p(lru))
        return sl, lru[:n].copy()


# ------------------------------------------------------------------ attend --
def attend(q: np.ndarray, window: np.ndarray, store: np.ndarray, kv_dtype: str,
           sel: np.ndarray, scale: float) -> np.ndarray:
    """q [Hq][D]; window [W][D]; store [cap][D]; sel [n] logical IDs -> out [Hq][D] f32."""
    q = _c(q, np.float32)
    Hq, D = q.shape
    window = _kv(window, kv_dtype)
    store = _kv(store, kv_dtype)
    sel = _c(sel, np.int32)
    W = window.shape[0] if window.size else 0
    out = np.zeros((Hq, D), np.float32)
    lib().oracle_attend(_p(q), Hq, D, _p(window), W, _p(store), DT[kv_dtype], _p(sel), sel.size,
                        float(scale), _p(out))
    return out


# ------------------------------------------------------------------ KVSwap --
def lowrank_score(U: np.ndarray, S: np.ndarray, V: np.ndarray, q: np.ndarray) -> np.ndarray:
    """U [T][r] f16 codes, S [r] f32, V [C][r] f16 codes, q [C] f32 -> score [T] f32."""
    U = _c(U, np.uint16)
    V = _c(V, np.uint16)
    S = _c(S, np.float32)
    q = _c(q, np.float32)
    T, r = U.shape
    C = V.shape[0]
    out = np.zeros(T, np.float32)
    lib().oracle_lowrank_score(_p(U), T, r, _p(S), _p(V), C, _p(q), _p(out))
    return out


def attend_kv(q: np.ndarray, K: np.ndarray, V: np.ndarray, kv_dtype: str, row_stride: int,
              pos: np.ndarray, scale: float) -> np.ndarray:
    """One head: q [dh]; K, V flat arrays where position p starts at p*row_stride."""
    q = _c(q, np.float32)
    K = _kv(K, kv_dtype)
    V = _kv(V, kv_dtype)
    pos = _c(pos, np.int32)
    out = np.zeros(q.size, np.float32)
    lib().oracle_attend_kv(_p(q), q.size, _p(K), _p(V), DT[kv_dtype], row_stride, _p(pos), pos.size,
                           float(scale), _p(out))
    return out


# ------------------------------------------------------------- decode step --
class DecodeState:
    """Oracle of whole decode steps for one workload: per sparse layer and
    sequence an LRU pool over a store of rows.

    store_rows[l][b] [cap][D] is the content of every entry; the first
    stored[l][b] entries (all of them by default) are stored up front, the rest
    by store() during decoding ([P1] store flow).

    step(predict=True) is a step on which the memory indexer fires: score the
    valid keys, select, then per layer map the selection to the layer's complete
    entries, stage them and attend.  step(predict=False) is a step of the
    decoding window the last prediction covers ([P2] LSA section: the indexer is
    triggered periodically and predicts the chunks of the coming short decoding
    window): no scoring, no staging; each layer attends over the entries it
    staged at the last prediction.  A stage that finds a never-stored entry
    ([P1] error 4) leaves its pool unchanged; that (layer, sequence) then has an
    empty list and attends to nothing (output 0) until the next prediction."""

    def __init__(self, wl, window_rows: List[List[np.ndarray]], store_rows: List[List[np.ndarray]],
                 stored: Optional[List[List[int]]] = None):
        # window_rows[layer][b] : [W][D]; store_rows[layer][b] : [cap][D] (kv dtype storage)
        self.wl = wl
        self.window_rows = window_rows
        # the caller's arrays, copied only when store() first changes one
        self.store_rows = [list(per_b) for per_b in store_rows]
        self._own = [[False] * len(per_b) for per_b in store_rows]
        row_bytes = wl.kv_dim * (4 if wl.kv_dtype == "f32" else 2)
        self.pools = []
        # the entries each (layer, sequence) staged at the last prediction, and
        # whether that stage failed (then the list is empty, window included)
        self.held = [[np.zeros(0, np.int32) for _ in range(wl.batch)] for _ in range(wl.n_layers)]
        self.failed = [[False] * wl.batch for _ in range(wl.n_layers)]
        for l in range(wl.n_layers):
            cap = wl.layer_cap(l)
            per_b = []
            for b in range(wl.batch):
                p = Pool(cap, wl.gpu_chunks, wl.window, row_bytes)
                p.set_replacement(self._weight(l), getattr(wl, "high_water", 100))
                n0 = cap if stored is None else int(stored[l][b])
                if n0 > 0:
                    p.store(0, n0)
                per_b.append(p)
            self.pools.append(per_b)

    def _weight(self, l: int) -> int:
        """Recency weight of layer l's pools: the workload's, for layers whose entries
        are the scored source entries; plain LRU elsewhere."""
        wl = self.wl
        return getattr(wl, "recency_w", 100) if wl.layer_ratios[l] == wl.src_ratio else 100

    def store(self, l: int, b: int, first: int, rows: np.ndarray) -> None:
        """[P1] store flow: entries first.. of layer l, sequence b get `rows` and are marked stored."""
        rows = np.asarray(rows)
        if not self._own[l][b]:
            self.store_rows[l][b] = np.array(self.store_rows[l][b], copy=True)
            self._own[l][b] = True
        self.store_rows[l][b][first:first + rows.shape[0]] = rows
        self.pools[l][b].store(first, rows.shape[0])

    def step(self, keys: Sequence[np.ndarray], q_idx: np.ndarray, w_idx: np.ndarray,
             q_attn: np.ndarray, k: Optional[int] = None, n_valid: Optional[Sequence[int]] = None,
             predict: bool = True) -> dict:
        """keys[b] [N][dk]; q_idx [B][n_idx][H][dk]; w_idx [B][n_idx][H]; q_attn [L][B][Hq][D];
        n_valid[b]: valid source entries (default: all of keys[b])."""
        wl = self.wl
        k = wl.k if k is None else k
        res = dict(scores=[], sel=[], layer_sel=[], phys=[], misses=[], status=[], out=[])
        if predict:
            for b in range(wl.batch):
                nv = None if n_valid is None else int(n_valid[b])
                e = score(keys[b], wl.key_dtype, q_idx[b], w_idx[b], wl.ensemble, n_valid=nv)
                s = select(e, wl.mode, k, wl.tau if wl.tau is not None else 0.5)
                res["scores"].append(e)
                res["sel"].append(s)
        for l in range(wl.n_layers):
            lsel, lphys, lmiss, lst, lout = [], [], [], [], []
            for b in range(wl.batch):
                st, phys, miss = 0, None, []
                if predict:
                    nv = res["scores"][b].size      # the valid entries that were scored
                    sl = ratio_map(res["sel"][b], wl.src_ratio, wl.layer_ratios[l], nv)
                    imp = None
                    if self._weight(l) < 100:
                        # the step's score of every entry; entries not scored rank lowest
                        imp = np.full(self.pools[l][b].cap, -np.inf, np.float32)
                        imp[:res["scores"][b].size] = res["scores"][b]
                    st, phys, miss = self.pools[l][b].stage(sl, imp)
                    if st != 0:
                        sl, phys, miss = np.zeros(0, np.int32), np.zeros(0, np.int32), []
                    self.held[l][b] = sl
                    self.failed[l][b] = st != 0
                sl = self.held[l][b]
                if self.failed[l][b]:
                    out = np.zeros((wl.hq, wl.kv_dim), np.float32)
                else:
                    out = attend(q_attn[l][b], self.window_rows[l][b], self.store_rows[l][b],
                                 wl.kv_dtype, sl, wl.scale)
                lsel.append(sl)
                lphys.append(phys)
                lmiss.append(miss)
                # on a window step, the status of the prediction it serves
                lst.append(ST_NOT_STORED if self.failed[l][b] else 0)
                lout.append(out)
            res["layer_sel"].append(lsel)
            res["phys"].append(lphys)
            res["misses"].append(lmiss)
            res["status"].append(lst)
            res["out"].append(lout)
        return res


# ------------------------------------------------------------ KVSwap step --
class KVSwapState:
    """Oracle of KVSwap decode steps for chosen segments (layer, group, b):
    low-rank score over all positions -> top-k (ties to the lowest position)
    -> the segment's LRU slot pool (window 0) -> per head attention over the
    full-precision K/V rows of the selected positions (read from the cold
    store by position, so it is also the reference with swapping off)."""

    def __init__(self, wl, segs):
        self.wl = wl
        self.segs = list(segs)
        row_bytes = wl.row_elems * 2
        self.pools = {}
        for seg in self.segs:
            p = Pool(wl.ctx, wl.slots, 0, row_bytes)
            p.store(0, wl.ctx)
            p.set_replacement(getattr(wl, "recency_w", 100), getattr(wl, "high_water", 100))
            self.pools[seg] = p

    def step(self, seg, U, S, V, q, cold) -> dict:
        """U [T][r] f16 codes, S [r] f32, V [C][r] f16 codes, q [C] f32, cold [T][2C] f16 codes
        -> dict(score, sel, phys, misses, out [heads][dh])."""
        wl = self.wl
        e = lowrank_score(U, S, V, q)
        sel = select(e, "topk", wl.k)
        st, phys, miss = self.pools[seg].stage(sel, e)
        if st != 0:
            raise RuntimeError(f"oracle stage status {st}")
        flat = np.ascontiguousarray(cold, dtype=np.uint16).reshape(-1)
        H, dh, C = wl.group_heads, wl.head_dim, wl.C
        out = np.zeros((H, dh), np.float32)
        for h in range(H):
            out[h] = attend_kv(q[h * dh:(h + 1) * dh], flat[h * dh:], flat[C + h * dh:], "f16", 2 * C, sel,
                               wl.scale)
        return dict(score=e, sel=sel, phys=phys, misses=miss, out=out)
