"""Thin ctypes binding of liblsa (include/lsa.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of liblsa.so.  Tensors are torch device tensors (PyTorch provides
device memory and streams); their data pointers and the current HIP stream
are passed straight to the C ABI.  If liblsa.so is missing this module raises
-- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblsa.so")

F32, BF16, F16, FP8_E4M3, MXFP4, MXINT8 = 0, 1, 2, 3, 4, 5
ENS = {"max": 0, "mean": 1}
MODE = {"topk": 0, "threshold": 1}
COLD = {"hbm": 0, "host": 1}
DTYPE = {"f32": F32, "bf16": BF16, "f16": F16, "fp8": FP8_E4M3, "mxfp4": MXFP4, "mxint8": MXINT8}
K_NAMES = ["score", "select", "stage", "gather", "attend", "combine"]
MAX_LAYERS = 64

STATUS = {0: "LSA_OK", 1: "LSA_ERR_INVALID_ARG", 2: "LSA_ERR_SLOTS_LT_TOPK", 3: "LSA_ERR_PINNED_CAP",
          4: "LSA_ERR_NOT_STORED", 5: "LSA_ERR_HIP", 6: "LSA_ERR_NO_MEMORY", 7: "LSA_ERR_UNSUPPORTED"}

P = ctypes.c_void_p
i32, i64, u64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_double


class LsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.msg = msg


class PoolDesc(ctypes.Structure):
    _fields_ = [("ctx", i64), ("ratio", i32), ("window", i32), ("gpu_chunks", i32), ("topk", i32),
                ("kv_dim", i32), ("batch", i32), ("dtype", i32), ("cold", i32), ("pinned_cap_bytes", u64),
                ("allow_topk_reduction", i32), ("kv_buf", P), ("kv_stride_b", i64),
                ("cold_buf", P), ("cold_stride_b", i64)]


class PoolStats(ctypes.Structure):
    _fields_ = [("hits", u64), ("misses", u64), ("h2d_bytes", u64), ("d2h_bytes", u64),
                ("compressed_cap", i64), ("swap_enabled", i32), ("resident", i32)]


class AdaptPolicy(ctypes.Structure):
    _fields_ = [("grow_miss_rate", f64), ("grow_h2d_bytes_per_step", f64), ("shrink_miss_rate", f64),
                ("step", i32), ("min_capacity", i32), ("max_capacity", i32)]


class StepDesc(ctypes.Structure):
    _fields_ = [("keys", P), ("key_dtype", i32), ("key_scales", P), ("n_keys", i64), ("n_valid", P), ("dk", i32),
                ("q_idx", P), ("w_idx", P), ("n_idx", i32), ("heads", i32), ("ensemble", i32),
                ("mode", i32), ("k", i32), ("tau", f64), ("src_ratio", i32),
                ("scores", P), ("sel", P), ("count", P),
                ("n_layers", i32), ("pools", P), ("q_attn", P), ("out", P), ("phys", P), ("n_rows", P),
                ("hq", i32), ("scale", f32), ("batch", i32)]


class KVSwapDesc(ctypes.Structure):
    _fields_ = [("U", P), ("S", P), ("V", P), ("factor_dtype", i32), ("T", i64), ("rank", i32),
                ("q", P), ("heads", i32), ("head_dim", i32), ("k", i32),
                ("scores", P), ("sel", P), ("count", P), ("n_pools", i32), ("pools", P),
                ("phys", P), ("n_rows", P), ("scale", f32), ("out", P)]


ABI_VERSION = 7

_SIGS = {
    "lsa_compressed_cap": (i64, [i64, i32]),
    "lsa_pinned_bytes": (u64, [i64, P, i32, i32, i32]),
    "lsa_max_capacity": (i32, [i32, i32]),
    "lsa_check_pinned": (i32, [i64, P, i32, i32, i32, u64]),
    "lsa_threshold_logit": (f32, [f64]),
    "lsa_status_string": (ctypes.c_char_p, [i32]),
    "lsa_last_error": (ctypes.c_char_p, []),
    "lsa_abi_version": (i32, []),
    "lsa_ctx_create": (i32, [ctypes.POINTER(P), i32]),
    "lsa_ctx_destroy": (None, [P]),
    "lsa_ctx_reserve": (i32, [P, u64]),
    "lsa_ctx_set_timing": (i32, [P, i32]),
    "lsa_ctx_set_key_policy": (i32, [P, i32]),
    "lsa_ctx_timing_read": (i32, [P, P, P]),
    "lsa_project": (i32, [P, i32, i32, P, P, i32, i32, i32, i32, P, P, P]),
    "lsa_score": (i32, [P, i32, P, i32, i64, P, i32, P, P, i32, i32, i32, P, P]),
    "lsa_select": (i32, [P, P, i32, i64, P, i32, i32, f64, P, P, P]),
    "lsa_pool_rows": (i64, [ctypes.POINTER(PoolDesc)]),
    "lsa_pool_create": (i32, [ctypes.POINTER(P), ctypes.POINTER(PoolDesc)]),
    "lsa_pool_destroy": (None, [P]),
    "lsa_pool_store": (i32, [P, i32, i64, i64, P, P]),
    "lsa_pool_host_rows": (P, [P, i32]),
    "lsa_pool_mark_stored": (i32, [P, i32, i64, i64, P]),
    "lsa_pool_reset": (i32, [P, P]),
    "lsa_pool_set_capacity": (i32, [P, i32, P]),
    "lsa_pool_capacity": (i32, [P]),
    "lsa_pool_set_replacement": (i32, [P, i32, i32]),
    "lsa_pool_adapt": (i32, [P, P, i32, P, P]),
    "lsa_pool_stats": (i32, [P, ctypes.POINTER(PoolStats), P]),
    "lsa_pool_state": (i32, [P, i32, P, P, ctypes.POINTER(i32), P]),
    "lsa_stage": (i32, [P, P, P, i32, i32, P, P, P, i32, P, P]),
    "lsa_attend": (i32, [P, P, P, i32, i64, i64, P, i32, P, i32, i32, i32, f32, P, P]),
    "lsa_decode_step": (i32, [P, ctypes.POINTER(StepDesc), P]),
    "lsa_decode_step_noalloc": (i32, [P, ctypes.POINTER(StepDesc), P]),
    "lsa_lookahead_prime": (i32, [P, ctypes.POINTER(StepDesc), P]),
    "lsa_lookahead_step": (i32, [P, ctypes.POINTER(StepDesc), P]),
    "lsa_lookahead_buffer": (i32, [P]),
    "lsa_decode_attend": (i32, [P, ctypes.POINTER(StepDesc), P]),
    "lsa_lookahead_attend": (i32, [P, ctypes.POINTER(StepDesc), P]),
    "lsa_score_lowrank": (i32, [P, P, i32, i32, i64, i32, P, P, i32, P, P, P]),
    "lsa_attend_kv": (i32, [P, P, P, i32, i64, i64, i32, i32, P, i32, P, i32, f32, P, P]),
    "lsa_kvswap_step": (i32, [P, ctypes.POINTER(KVSwapDesc), P]),
}
EXPORTS = tuple(_SIGS)

_lib = None


def lib():
    """Load liblsa.so (built by learned_sparse_kv_amd/build.py); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(st: int) -> None:
    if st != 0:
        raise LsaError(st, lib().lsa_last_error().decode(errors="replace"))


# --------------------------------------------------------------- helpers
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _host_i64(vals) -> Optional[ctypes.Array]:
    if vals is None:
        return None
    arr = (i64 * len(vals))(*[int(v) for v in vals])
    return arr


def row_dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    if t.dtype == torch.float4_e2m1fn_x2:
        return MXFP4
    if t.dtype == torch.int8:
        return MXINT8
    raise ValueError(f"unsupported dtype {t.dtype}")


# ----------------------------------------------------------- closed forms
def compressed_cap(ctx: int, ratio: int) -> int:
    return int(lib().lsa_compressed_cap(ctx, ratio))


def pinned_bytes(ctx: int, ratios: Sequence[int], kv_dim: int, dtype: int = F32) -> int:
    r = (i32 * len(ratios))(*ratios)
    return int(lib().lsa_pinned_bytes(ctx, ctypes.cast(r, P), len(ratios), kv_dim, dtype))


def max_capacity(window: int, gpu_chunks: int) -> int:
    return int(lib().lsa_max_capacity(window, gpu_chunks))


def check_pinned(ctx: int, ratios: Sequence[int], kv_dim: int, dtype: int, cap_bytes: int) -> None:
    r = (i32 * len(ratios))(*ratios)
    _check(lib().lsa_check_pinned(ctx, ctypes.cast(r, P), len(ratios), kv_dim, dtype, cap_bytes))


def threshold_logit(tau: float) -> float:
    return float(lib().lsa_threshold_logit(tau))


# ------------------------------------------------------------------ ctx
class Ctx:
    def __init__(self, device: int = 0):
        h = P()
        _check(lib().lsa_ctx_create(ctypes.byref(h), device))
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            lib().lsa_ctx_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reserve(self, nbytes: int):
        _check(lib().lsa_ctx_reserve(self.h, nbytes))

    def set_timing(self, on: bool):
        _check(lib().lsa_ctx_set_timing(self.h, 1 if on else 0))

    def set_key_policy(self, non_temporal: bool):
        _check(lib().lsa_ctx_set_key_policy(self.h, 1 if non_temporal else 0))

    def timing_read(self) -> dict:
        ms = (f64 * 6)()
        n = (i64 * 6)()
        _check(lib().lsa_ctx_timing_read(self.h, ctypes.cast(ms, P), ctypes.cast(n, P)))
        return {K_NAMES[i]: (ms[i], n[i]) for i in range(6)}


# ----------------------------------------------------------- projection
def project(hidden, wq, ww, q, w, stream=None) -> None:
    """hidden [B][d_model] f32, wq [n_idx][H][dk][d_model] and ww [n_idx][H][d_model]
    (f32/bf16) -> q [B][n_idx][H][dk] f32, w [B][n_idx][H] f32."""
    for t, n in ((hidden, "hidden"), (wq, "wq"), (ww, "ww"), (q, "q"), (w, "w")):
        _dev(t, n)
    B, d_model = hidden.shape
    n_idx, H, dk, d2 = wq.shape
    if d2 != d_model or tuple(ww.shape) != (n_idx, H, d_model) or ww.dtype != wq.dtype:
        raise ValueError("projection weight shapes or dtypes do not match")
    if tuple(q.shape) != (B, n_idx, H, dk) or tuple(w.shape) != (B, n_idx, H):
        raise ValueError("projection output shapes do not match")
    _check(lib().lsa_project(_ptr(hidden), B, d_model, _ptr(wq), _ptr(ww), row_dtype_code(wq), n_idx, H, dk,
                             _ptr(q), _ptr(w), _stream(stream)))


# ---------------------------------------------------------------- score
def _keys_args(keys, key_scales, dk: int):
    """(dtype code, key_scales pointer) after checking the key and scale shapes: keys
    [B][N][dk] (f32, bf16, fp8 e4m3fn or int8 = MX INT8) or [B][N][dk/2]
    (float4_e2m1fn_x2 = MX FP4); MX keys need key_scales [B][N][dk/32] (one byte each)."""
    code = row_dtype_code(keys)
    B, N, width = keys.shape
    if width != (dk // 2 if code == MXFP4 else dk):
        raise ValueError(f"keys' last dimension {width} does not match dk {dk}")
    if code in (MXFP4, MXINT8):
        if key_scales is None:
            raise ValueError("MX keys need key_scales")
        _dev(key_scales, "key_scales")
        if tuple(key_scales.shape) != (B, N, dk // 32) or key_scales.element_size() != 1:
            raise ValueError("key_scales must be one byte per 32 key elements, [B][N][dk/32]")
        return code, _ptr(key_scales)
    return code, None


def score(keys, q, w, scores, ensemble: str = "max", n_valid=None, stream=None, key_scales=None) -> None:
    """keys [B][N][dk] (or [B][N][dk/2] MX FP4), q [B][n_idx][H][dk] f32, w [B][n_idx][H] f32
    -> scores [B][N] f32."""
    _dev(keys, "keys"), _dev(q, "q"), _dev(w, "w"), _dev(scores, "scores")
    B, n_idx, H, dk = q.shape
    N = keys.shape[1]
    code, sp = _keys_args(keys, key_scales, dk)
    nv = _host_i64(n_valid)
    _check(lib().lsa_score(_ptr(keys), code, sp, B, N, ctypes.cast(nv, P) if nv else None, dk,
                           _ptr(q), _ptr(w), n_idx, H, ENS[ensemble], _ptr(scores), _stream(stream)))


def select(ctx: Ctx, scores, k: int, sel, count, mode: str = "topk", tau: float = 0.5, n_valid=None,
           stream=None) -> None:
    """scores [n_seg][N] f32 -> sel [n_seg][k] i32 (ascending, -1 padded), count [n_seg] i32."""
    _dev(scores, "scores"), _dev(sel, "sel"), _dev(count, "count")
    n_seg, N = scores.shape
    nv = _host_i64(n_valid)
    _check(lib().lsa_select(ctx.h, _ptr(scores), n_seg, N, ctypes.cast(nv, P) if nv else None, MODE[mode], k,
                            float(tau), _ptr(sel), _ptr(count), _stream(stream)))


# ----------------------------------------------------------------- pools
class Pool:
    """One sparse layer's slot pool for `batch` sequences (lsa_pool)."""

    def __init__(self, ctx: int, ratio: int, kv_buf, window: int, gpu_chunks: int, topk: int,
                 kv_dim: int = 512, batch: int = 1, cold: str = "hbm", pinned_cap_bytes: int = 0,
                 allow_topk_reduction: bool = False, kv_stride_b: Optional[int] = None,
                 cold_buf=None, cold_stride_b: int = 0):
        """cold_buf: optional caller-owned device tensor holding the cold rows of
        every sequence (sequence b at byte offset b * cold_stride_b)."""
        _dev(kv_buf, "kv_buf")
        d = PoolDesc()
        d.ctx, d.ratio, d.window, d.gpu_chunks, d.topk = ctx, ratio, window, gpu_chunks, topk
        d.kv_dim, d.batch, d.dtype, d.cold = kv_dim, batch, row_dtype_code(kv_buf), COLD[cold]
        d.pinned_cap_bytes = pinned_cap_bytes
        d.allow_topk_reduction = 1 if allow_topk_reduction else 0
        d.kv_buf = _ptr(kv_buf)
        if cold_buf is not None:
            if not cold_buf.is_cuda:
                raise ValueError("cold_buf must be a device tensor")
            d.cold_buf, d.cold_stride_b = cold_buf.data_ptr(), cold_stride_b
        self.cold_buf = cold_buf  # keep the caller's buffer alive
        rows = int(lib().lsa_pool_rows(ctypes.byref(d)))
        d.kv_stride_b = kv_stride_b if kv_stride_b is not None else rows * kv_dim
        if kv_buf.numel() < batch * d.kv_stride_b and batch > 0:
            raise ValueError(f"kv_buf holds {kv_buf.numel()} elements, needs {batch * d.kv_stride_b}")
        self.desc = d
        self.kv_buf = kv_buf  # keep the caller's buffer alive
        self.rows = rows
        self.cap = compressed_cap(ctx, ratio)
        self.swap = self.cap > gpu_chunks
        self.batch = batch
        self.kv_dim = kv_dim
        self.window = window
        self.gpu_chunks = gpu_chunks
        h = P()
        _check(lib().lsa_pool_create(ctypes.byref(h), ctypes.byref(d)))
        self.h = h

    @staticmethod
    def rows_needed(ctx: int, ratio: int, window: int, gpu_chunks: int) -> int:
        d = PoolDesc()
        d.ctx, d.ratio, d.window, d.gpu_chunks = ctx, ratio, window, gpu_chunks
        return int(lib().lsa_pool_rows(ctypes.byref(d)))

    def close(self):
        if getattr(self, "h", None):
            lib().lsa_pool_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def store(self, b: int, first: int, rows, stream=None) -> None:
        """rows: a device tensor or a C-contiguous numpy array [count][kv_dim] in the pool dtype."""
        if isinstance(rows, np.ndarray):
            rows = np.ascontiguousarray(rows)
            ptr, count = rows.ctypes.data, rows.shape[0]
        else:
            _dev(rows, "rows")
            ptr, count = _ptr(rows), rows.shape[0]
        _check(lib().lsa_pool_store(self.h, b, first, count, ptr, _stream(stream)))

    def host_rows(self, b: int, np_dtype=np.float32) -> Optional[np.ndarray]:
        """numpy view of sequence b's pinned cold pool [cap][kv_dim] (host cold pools only)."""
        p = lib().lsa_pool_host_rows(self.h, b)
        if not p:
            return None
        item = np.dtype(np_dtype).itemsize
        n = self.cap * self.kv_dim
        buf = (ctypes.c_char * (n * item)).from_address(p)
        return np.frombuffer(buf, dtype=np_dtype).reshape(self.cap, self.kv_dim)

    def mark_stored(self, b: int, first: int, count: int, stream=None) -> None:
        _check(lib().lsa_pool_mark_stored(self.h, b, first, count, _stream(stream)))

    def set_capacity(self, capacity: int, stream=None) -> None:
        """Slots the pool may use (lsa_pool_set_capacity): grow, or shrink keeping the most recent entries."""
        _check(lib().lsa_pool_set_capacity(self.h, int(capacity), _stream(stream)))

    def capacity(self) -> int:
        return int(lib().lsa_pool_capacity(self.h))

    def set_replacement(self, recency_weight: int = 100, high_water: int = 100) -> None:
        """Replacement weighing recency against importance, and the high-water mark (lsa_pool_set_replacement)."""
        _check(lib().lsa_pool_set_replacement(self.h, int(recency_weight), int(high_water)))

    def adapt(self, steps: int, min_capacity: int, max_capacity: int, step: int, grow_miss_rate: float = 0.5,
              grow_h2d_bytes_per_step: float = 10e6, shrink_miss_rate: float = 0.0, stream=None) -> int:
        """Adaptive capacity from the counters since the last call (lsa_pool_adapt); -> the new capacity."""
        pol = AdaptPolicy(float(grow_miss_rate), float(grow_h2d_bytes_per_step), float(shrink_miss_rate), int(step),
                          int(min_capacity), int(max_capacity))
        out = ctypes.c_int32(0)
        _check(lib().lsa_pool_adapt(self.h, ctypes.byref(pol), int(steps), ctypes.byref(out), _stream(stream)))
        return int(out.value)

    def reset(self, stream=None) -> None:
        _check(lib().lsa_pool_reset(self.h, _stream(stream)))

    def stats(self, stream=None) -> dict:
        s = PoolStats()
        st = lib().lsa_pool_stats(self.h, ctypes.byref(s), _stream(stream))
        out = dict(hits=s.hits, misses=s.misses, h2d_bytes=s.h2d_bytes, d2h_bytes=s.d2h_bytes,
                   compressed_cap=s.compressed_cap, swap_enabled=bool(s.swap_enabled), resident=s.resident)
        _check(st)
        return out

    def state(self, b: int, stream=None):
        """-> (slot_logical [S] int32, lru slot ids most- to least-recent)."""
        S = self.gpu_chunks
        sl = np.zeros(S, np.int32)
        lr = np.zeros(S, np.int32)
        n = i32(0)
        _check(lib().lsa_pool_state(self.h, b, sl.ctypes.data, lr.ctypes.data, ctypes.byref(n), _stream(stream)))
        return sl, lr[:n.value].copy()


def stage(pool: Pool, sel, count, src_ratio: int, phys, n_rows, n_valid=None, importance=None,
          stream=None) -> None:
    """sel [B][k] i32, count [B] i32 -> phys [B][window + k] i32, n_rows [B] i32; n_valid:
    valid source entries per sequence (None: every chunk complete); importance [B][cap] f32
    for a pool that weighs importance in its replacement."""
    _dev(sel, "sel"), _dev(count, "count"), _dev(phys, "phys"), _dev(n_rows, "n_rows")
    if importance is not None:
        _dev(importance, "importance")
    nv = _host_i64(n_valid)
    _check(lib().lsa_stage(pool.h, _ptr(sel), _ptr(count), sel.shape[1], src_ratio,
                           ctypes.cast(nv, P) if nv else None, _ptr(importance), _ptr(phys), phys.shape[1],
                           _ptr(n_rows), _stream(stream)))


def attend(ctx: Ctx, q, kv, phys, n_rows, out, scale: float, kv_rows: Optional[int] = None,
           kv_stride_b: Optional[int] = None, stream=None) -> None:
    """q [B][hq][D] f32; kv [B][rows][D]; phys [B][stride] i32; n_rows [B] i32 -> out [B][hq][D] f32."""
    _dev(q, "q"), _dev(kv, "kv"), _dev(phys, "phys"), _dev(n_rows, "n_rows"), _dev(out, "out")
    B, hq, D = q.shape
    rows = kv.shape[1] if kv_rows is None else kv_rows
    stride = kv.shape[1] * kv.shape[2] if kv_stride_b is None else kv_stride_b
    _check(lib().lsa_attend(ctx.h, _ptr(q), _ptr(kv), row_dtype_code(kv), stride, rows, _ptr(phys), phys.shape[1],
                            _ptr(n_rows), B, hq, D, float(scale), _ptr(out), _stream(stream)))


def _step_desc(keys, q_idx, w_idx, pools, q_attn, out, scores, sel, count, k, src_ratio, scale, ensemble="max",
               mode="topk", tau=0.5, n_valid=None, phys=None, n_rows=None, key_scales=None):
    for t, n in ((keys, "keys"), (q_idx, "q_idx"), (w_idx, "w_idx"), (q_attn, "q_attn"), (out, "out"),
                 (scores, "scores"), (sel, "sel"), (count, "count")):
        _dev(t, n)
    B, n_idx, H, dk = q_idx.shape
    N = keys.shape[1]
    code, sp = _keys_args(keys, key_scales, dk)
    L, _, hq, D = q_attn.shape
    if L != len(pools):
        raise ValueError("q_attn's first dimension must equal the number of pools")
    d = StepDesc()
    nv = _host_i64(n_valid)
    pool_arr = (P * len(pools))(*[p.h for p in pools])
    d.keys, d.key_dtype, d.key_scales, d.n_keys, d.n_valid, d.dk = _ptr(keys), code, sp, N, \
        (ctypes.cast(nv, P) if nv else None), dk
    d.q_idx, d.w_idx, d.n_idx, d.heads, d.ensemble = _ptr(q_idx), _ptr(w_idx), n_idx, H, ENS[ensemble]
    d.mode, d.k, d.tau, d.src_ratio = MODE[mode], k, float(tau), src_ratio
    d.scores, d.sel, d.count = _ptr(scores), _ptr(sel), _ptr(count)
    d.n_layers, d.pools, d.q_attn, d.out = len(pools), ctypes.cast(pool_arr, P), _ptr(q_attn), _ptr(out)
    d.phys = _ptr(phys) if phys is not None else None
    d.n_rows = _ptr(n_rows) if n_rows is not None else None
    d.hq, d.scale, d.batch = hq, float(scale), B
    return d, (nv, pool_arr)


def lookahead_prime(ctx: Ctx, *, keys, q_idx, w_idx, pools: Sequence[Pool], q_attn, out, scores, sel, count,
                    k: int, src_ratio: int, scale: float, ensemble: str = "max", mode: str = "topk",
                    tau: float = 0.5, n_valid=None, phys=None, n_rows=None, stream=None, key_scales=None) -> None:
    """Stage the rows of the first lookahead step (lsa_lookahead_prime); arguments as decode_step,
    with phys [2][L][B][window + k] and n_rows [2][L][B] when given."""
    d, keep = _step_desc(keys, q_idx, w_idx, pools, q_attn, out, scores, sel, count, k, src_ratio, scale, ensemble,
                         mode, tau, n_valid, phys, n_rows, key_scales)
    _check(lib().lsa_lookahead_prime(ctx.h, ctypes.byref(d), _stream(stream)))


def lookahead_step(ctx: Ctx, *, keys, q_idx, w_idx, pools: Sequence[Pool], q_attn, out, scores, sel, count,
                   k: int, src_ratio: int, scale: float, ensemble: str = "max", mode: str = "topk",
                   tau: float = 0.5, n_valid=None, phys=None, n_rows=None, stream=None, key_scales=None) -> None:
    """Attend this step (q_attn -> out) while predicting and staging the next one from q_idx / w_idx
    (lsa_lookahead_step)."""
    d, keep = _step_desc(keys, q_idx, w_idx, pools, q_attn, out, scores, sel, count, k, src_ratio, scale, ensemble,
                         mode, tau, n_valid, phys, n_rows, key_scales)
    _check(lib().lsa_lookahead_step(ctx.h, ctypes.byref(d), _stream(stream)))


class PreparedStep:
    """A step descriptor marshalled once and launched many times (the tensors it
    points at must stay alive and keep their addresses)."""

    def __init__(self, fn_name: str, ctx: Ctx, stream=None, **kw):
        self.desc, self._keep = _step_desc(**kw)
        self._fn = getattr(lib(), fn_name)
        self._ctx = ctx.h
        self._ref = ctypes.byref(self.desc)
        self._stream = _stream(stream)

    def __call__(self) -> None:
        _check(self._fn(self._ctx, self._ref, self._stream))


def lookahead_attend(ctx: Ctx, *, keys, q_idx, w_idx, pools: Sequence[Pool], q_attn, out, scores, sel, count,
                     k: int, src_ratio: int, scale: float, ensemble: str = "max", mode: str = "topk",
                     tau: float = 0.5, n_valid=None, phys=None, n_rows=None, stream=None, key_scales=None) -> None:
    """Attend this step over the current prediction's rows without predicting (lsa_lookahead_attend)."""
    d, keep = _step_desc(keys, q_idx, w_idx, pools, q_attn, out, scores, sel, count, k, src_ratio, scale, ensemble,
                         mode, tau, n_valid, phys, n_rows, key_scales)
    _check(lib().lsa_lookahead_attend(ctx.h, ctypes.byref(d), _stream(stream)))


def lookahead_buffer(ctx: Ctx) -> int:
    return int(lib().lsa_lookahead_buffer(ctx.h))


def decode_step(ctx: Ctx, *, keys, q_idx, w_idx, pools: Sequence[Pool], q_attn, out, scores, sel, count,
                k: int, src_ratio: int, scale: float, ensemble: str = "max", mode: str = "topk",
                tau: float = 0.5, n_valid=None, phys=None, n_rows=None, stream=None, key_scales=None) -> None:
    """One LSA decode step over len(pools) sparse layers (lsa_decode_step).

    keys [B][N][dk] (MX FP4: [B][N][dk/2]) with key_scales [B][N][dk/32] for the MX dtypes;
    q_idx [B][n_idx][H][dk]; w_idx [B][n_idx][H]; q_attn / out [L][B][hq][D] f32;
    scores [B][N] f32; sel [B][k] i32; count [B] i32; phys [L][B][window + k] i32 and
    n_rows [L][B] i32 optional."""
    d, keep = _step_desc(keys, q_idx, w_idx, pools, q_attn, out, scores, sel, count, k, src_ratio, scale, ensemble,
                         mode, tau, n_valid, phys, n_rows, key_scales)
    _check(lib().lsa_decode_step(ctx.h, ctypes.byref(d), _stream(stream)))


def decode_step_noalloc(ctx: Ctx, *, keys, q_idx, w_idx, pools: Sequence[Pool], q_attn, out, scores, sel, count,
                        k: int, src_ratio: int, scale: float, ensemble: str = "max", mode: str = "topk",
                        tau: float = 0.5, n_valid=None, phys=None, n_rows=None, stream=None,
                        key_scales=None) -> None:
    """decode_step with its scratch in the library's static device array (lsa_decode_step_noalloc)."""
    d, keep = _step_desc(keys, q_idx, w_idx, pools, q_attn, out, scores, sel, count, k, src_ratio, scale, ensemble,
                         mode, tau, n_valid, phys, n_rows, key_scales)
    _check(lib().lsa_decode_step_noalloc(ctx.h, ctypes.byref(d), _stream(stream)))


def decode_attend(ctx: Ctx, *, keys, q_idx, w_idx, pools: Sequence[Pool], q_attn, out, scores, sel, count,
                  k: int, src_ratio: int, scale: float, ensemble: str = "max", mode: str = "topk",
                  tau: float = 0.5, n_valid=None, phys=None, n_rows=None, stream=None, key_scales=None) -> None:
    """Attend over the rows the last decode_step staged (lsa_decode_attend): a step of the
    decoding window a periodic prediction serves."""
    d, keep = _step_desc(keys, q_idx, w_idx, pools, q_attn, out, scores, sel, count, k, src_ratio, scale, ensemble,
                         mode, tau, n_valid, phys, n_rows, key_scales)
    _check(lib().lsa_decode_attend(ctx.h, ctypes.byref(d), _stream(stream)))


# ---------------------------------------------------------------- KVSwap
def score_lowrank(ctx: Ctx, U, S, V, q, scores, stream=None) -> None:
    """U [n_seg][T][r] f16, S [n_seg][r] f32, V [n_seg][C][r] f16, q [n_seg][C] f32 -> scores [n_seg][T] f32."""
    for t, n in ((U, "U"), (S, "S"), (V, "V"), (q, "q"), (scores, "scores")):
        _dev(t, n)
    n_seg, T, r = U.shape
    C = V.shape[1]
    _check(lib().lsa_score_lowrank(ctx.h, _ptr(U), row_dtype_code(U), n_seg, T, r, _ptr(S), _ptr(V), C, _ptr(q),
                                   _ptr(scores), _stream(stream)))


def attend_kv(ctx: Ctx, q, kv, phys, n_rows, out, scale: float, kv_rows: Optional[int] = None,
              kv_stride_seg: Optional[int] = None, stream=None) -> None:
    """q [n_seg][heads][dh] f32; kv [n_seg][rows][2*heads*dh] f16/bf16; phys [n_seg][stride] i32;
    n_rows [n_seg] i32 -> out [n_seg][heads][dh] f32."""
    for t, n in ((q, "q"), (kv, "kv"), (phys, "phys"), (n_rows, "n_rows"), (out, "out")):
        _dev(t, n)
    n_seg, heads, dh = q.shape
    rows = kv.shape[1] if kv_rows is None else kv_rows
    stride = kv.shape[1] * kv.shape[2] if kv_stride_seg is None else kv_stride_seg
    _check(lib().lsa_attend_kv(ctx.h, _ptr(q), _ptr(kv), row_dtype_code(kv), stride, rows, heads, dh, _ptr(phys),
                               phys.shape[1], _ptr(n_rows), n_seg, float(scale), _ptr(out), _stream(stream)))


def kvswap_step(ctx: Ctx, *, U, S, V, q, pools: Sequence[Pool], k: int, heads: int, head_dim: int, scores, sel,
                count, phys, n_rows, out, scale: float, stream=None) -> None:
    """One KVSwap decode step (lsa_kvswap_step); segment s = pool * batch + b.

    U [n_seg][T][r] f16; S [n_seg][r]; V [n_seg][C][r] f16; q [n_seg][C] f32; scores [n_seg][T] f32 or
    None (score and top-k in one launch, no scores written); sel / phys [n_seg][k] i32; count / n_rows
    [n_seg] i32; out [n_seg][heads][head_dim] f32."""
    for t, n in ((U, "U"), (S, "S"), (V, "V"), (q, "q"), (sel, "sel"), (count, "count"),
                 (phys, "phys"), (n_rows, "n_rows"), (out, "out")):
        _dev(t, n)
    if scores is not None:
        _dev(scores, "scores")
    n_seg, T, r = U.shape
    d = KVSwapDesc()
    pool_arr = (P * len(pools))(*[p.h for p in pools])
    d.U, d.S, d.V, d.factor_dtype, d.T, d.rank = _ptr(U), _ptr(S), _ptr(V), row_dtype_code(U), T, r
    d.q, d.heads, d.head_dim, d.k = _ptr(q), heads, head_dim, k
    d.scores, d.sel, d.count = _ptr(scores), _ptr(sel), _ptr(count)
    d.n_pools, d.pools = len(pools), ctypes.cast(pool_arr, P)
    d.phys, d.n_rows, d.scale, d.out = _ptr(phys), _ptr(n_rows), float(scale), _ptr(out)
    _check(lib().lsa_kvswap_step(ctx.h, ctypes.byref(d), _stream(stream)))
