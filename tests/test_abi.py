"""CPU tests of the C-ABI library: it loads, exports every function that
include/lsa.h declares, and its host-only logic (closed forms, argument
validation, the page's start-up errors) behaves as specified.  No kernel runs."""
import ctypes
import os
import re

import pytest

import oracle
from learned_sparse_kv_amd import lsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "lsa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    L = lsa.lib()
    names = declared_functions()
    assert len(names) >= 25
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(lsa.EXPORTS)
    assert L.lsa_abi_version() == lsa.ABI_VERSION == 7


def test_closed_forms_match_oracle():
    for ctx in (0, 1, 63, 64, 65, 8192, 262144, 1048576, 1000003):
        for r in (1, 4, 128):
            assert lsa.compressed_cap(ctx, r) == oracle.compressed_cap(ctx, r)
    ratios = [4] * 20 + [128] * 21
    for ctx in (8192, 262144, 1048576):
        assert lsa.pinned_bytes(ctx, ratios, 512) == oracle.pinned_bytes(ctx, ratios, 512, 4)
        assert lsa.pinned_bytes(ctx, ratios, 512, lsa.BF16) == oracle.pinned_bytes(ctx, ratios, 512, 2)
    assert lsa.max_capacity(128, 512) == 640
    assert lsa.compressed_cap(-1, 4) == -1 and lsa.compressed_cap(10, 0) == -1


def test_threshold_logit_matches_oracle():
    for tau in (1e-9, 0.01, 0.3, 0.5, 0.73, 0.9, 0.999999, 1 - 1e-12):
        assert lsa.threshold_logit(tau) == float(oracle.threshold_float(tau))
    import math
    assert math.isnan(lsa.threshold_logit(0.0)) and math.isnan(lsa.threshold_logit(1.0))


def test_pinned_cap_error_message():
    # page 1, error 3: "pinned cache exceeds cap: required_mib=XXX cap_mib=YYY"
    ratios = [4] * 20 + [128] * 21
    lsa.check_pinned(1048576, ratios, 512, lsa.F32, 16384 << 20)
    with pytest.raises(lsa.LsaError) as e:
        lsa.check_pinned(1048576, ratios, 512, lsa.F32, 1024 << 20)
    assert e.value.status == 3
    assert "required_mib=10576" in e.value.msg and "cap_mib=1024" in e.value.msg


def _desc(**kw):
    d = lsa.PoolDesc()
    d.ctx, d.ratio, d.window, d.gpu_chunks, d.topk, d.kv_dim, d.batch = 8192, 4, 128, 512, 512, 512, 1
    d.dtype, d.cold, d.pinned_cap_bytes, d.allow_topk_reduction = 0, 0, 0, 0
    d.kv_buf, d.kv_stride_b = 0x1000, 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _create(d):
    h = ctypes.c_void_p()
    st = lsa.lib().lsa_pool_create(ctypes.byref(h), ctypes.byref(d))
    return st, lsa.lib().lsa_last_error().decode()


def test_pool_validation_errors_before_any_device_call():
    # page 1, error 2: GPU_CHUNKS must be >= index_topk (unless the test override)
    st, msg = _create(_desc(gpu_chunks=256, topk=512))
    assert st == 2 and "index_topk" in msg
    # page 1, error 3 for a pinned-host cold pool
    st, msg = _create(_desc(cold=1, pinned_cap_bytes=1 << 20))
    assert st == 3 and "required_mib=4" in msg and "cap_mib=1" in msg
    # invalid arguments
    assert _create(_desc(kv_buf=None))[0] == 1
    assert _create(_desc(gpu_chunks=0))[0] == 1
    assert _create(_desc(ctx=1 << 20, gpu_chunks=5000, topk=512))[0] == 7
    assert _create(_desc(topk=2000))[0] == 1
    assert _create(_desc(batch=0))[0] == 1
    assert _create(_desc(dtype=9))[0] == 7
    assert _create(_desc(dtype=lsa.FP8_E4M3))[0] == 7   # fp8 is for indexer keys only
    # a caller-owned cold store must be device memory and hold every sequence
    assert _create(_desc(cold=1, cold_buf=0x2000))[0] == 1
    st, msg = _create(_desc(batch=2, kv_stride_b=1 << 20, cold_buf=0x2000, cold_stride_b=1024))
    assert st == 1 and "cold_stride_b" in msg


def test_kvswap_argument_checks():
    L = lsa.lib()
    ctx = 0x10   # never dereferenced: every call below is rejected before using it
    # lsa_score_lowrank(ctx, U, dtype, n_seg, T, rank, S, V, C, q, scores, stream)
    assert L.lsa_score_lowrank(None, 0x10, 2, 1, 64, 32, 0x10, 0x10, 512, 0x10, 0x10, None) == 1
    assert L.lsa_score_lowrank(ctx, None, 2, 1, 64, 32, 0x10, 0x10, 512, 0x10, 0x10, None) == 1
    assert L.lsa_score_lowrank(ctx, 0x10, 0, 1, 64, 32, 0x10, 0x10, 512, 0x10, 0x10, None) == 7
    assert L.lsa_score_lowrank(ctx, 0x10, 2, 1, 64, 24, 0x10, 0x10, 512, 0x10, 0x10, None) == 7
    assert L.lsa_score_lowrank(ctx, 0x10, 2, 1, 64, 32, 0x10, 0x10, 5000, 0x10, 0x10, None) == 7
    assert L.lsa_score_lowrank(ctx, 0x10, 2, 1, 1 << 27, 32, 0x10, 0x10, 512, 0x10, 0x10, None) == 7
    # lsa_attend_kv(ctx, q, kv, dtype, kv_stride_seg, kv_rows, heads, dh, phys, phys_stride, n_rows, n_seg, scale, out, s)
    args = [ctx, 0x10, 0x10, 2, 1 << 20, 400, 4, 128, 0x10, 400, 0x10, 2, 0.1, 0x10, None]

    def akv(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.lsa_attend_kv(*a)
    assert akv(a0=None) == 1
    assert akv(a3=0) == 7            # f32 rows
    assert akv(a6=9) == 7            # heads
    assert akv(a7=96) == 7           # head_dim
    assert akv(a9=5000) == 1         # phys_stride
    assert akv(a4=1000) == 1         # kv_stride_seg below kv_rows * row elements
    assert akv(a12=float("nan")) == 1
    assert L.lsa_kvswap_step(None, None, None) == 1
    d = lsa.KVSwapDesc()
    assert L.lsa_kvswap_step(ctx, ctypes.byref(d), None) == 1   # no pools


def test_context_setters_reject_null():
    L = lsa.lib()
    assert L.lsa_ctx_set_key_policy(None, 1) == 1
    assert L.lsa_ctx_set_timing(None, 1) == 1


def test_pool_rows_swap_auto_disable():
    # page 1 troubleshooting: 64 tokens at ratio 4 -> cap 16; gpu_chunks >= 16 keeps it resident
    assert lsa.Pool.rows_needed(64, 4, 128, 16) == 128 + 16
    assert lsa.Pool.rows_needed(64, 4, 128, 64) == 128 + 16
    assert lsa.Pool.rows_needed(64, 4, 128, 8) == 128 + 8
    assert lsa.Pool.rows_needed(1048576, 4, 128, 1024) == 128 + 1024


def test_score_and_select_argument_checks():
    L = lsa.lib()
    # dk unsupported / heads too many / bad ensemble: rejected on the host
    assert L.lsa_score(0x10, 0, None, 1, 100, None, 48, 0x10, 0x10, 1, 4, 0, 0x10, None) == 7
    assert L.lsa_score(0x10, 0, None, 1, 100, None, 64, 0x10, 0x10, 1, 9, 0, 0x10, None) == 7
    assert L.lsa_score(0x10, 0, None, 1, 100, None, 64, 0x10, 0x10, 1, 4, 5, 0x10, None) == 1
    assert L.lsa_score(None, 0, None, 1, 100, None, 64, 0x10, 0x10, 1, 4, 0, 0x10, None) == 1
    # projection: d_model a multiple of 8, batch in range, f32/bf16 weights, aligned hidden
    assert L.lsa_project(0x10, 1, 4100, 0x10, 0x10, 1, 3, 8, 128, 0x10, 0x10, None) == 7
    assert L.lsa_project(0x10, 0, 4096, 0x10, 0x10, 1, 3, 8, 128, 0x10, 0x10, None) == 1
    assert L.lsa_project(0x10, 1, 4096, 0x10, 0x10, lsa.FP8_E4M3, 3, 8, 128, 0x10, 0x10, None) == 7
    assert L.lsa_project(0x14, 1, 4096, 0x10, 0x10, 1, 3, 8, 128, 0x10, 0x10, None) == 1
    assert L.lsa_project(None, 1, 4096, 0x10, 0x10, 1, 3, 8, 128, 0x10, 0x10, None) == 1
    # key dtypes: f32, bf16 and fp8 E4M3; f16 keys and unknown codes are unsupported
    assert L.lsa_score(0x10, lsa.F16, None, 1, 100, None, 64, 0x10, 0x10, 1, 4, 0, 0x10, None) == 7
    assert L.lsa_score(0x10, 9, None, 1, 100, None, 64, 0x10, 0x10, 1, 4, 0, 0x10, None) == 7
    # MX keys need their block scales, and MX FP4 needs dk >= 64
    assert L.lsa_score(0x10, lsa.MXFP4, None, 1, 100, None, 128, 0x10, 0x10, 1, 4, 0, 0x10, None) == 1
    assert L.lsa_score(0x10, lsa.MXINT8, None, 1, 100, None, 128, 0x10, 0x10, 1, 4, 0, 0x10, None) == 1
    assert L.lsa_score(0x10, lsa.MXFP4, 0x10, 1, 100, None, 32, 0x10, 0x10, 1, 4, 0, 0x10, None) == 7
    assert L.lsa_score(0x10, 6, 0x10, 1, 100, None, 128, 0x10, 0x10, 1, 4, 0, 0x10, None) == 7
    # a sequence's keys must stay under 4 GiB: 2^25 keys x 128 bytes is the limit for fp8
    assert L.lsa_score(0x10, lsa.FP8_E4M3, None, 1, 1 << 25, None, 128, 0x10, 0x10, 1, 4, 0, 0x10, None) == 7
    assert L.lsa_select(None, 0x10, 1, 100, None, 0, 8, 0.5, 0x10, 0x10, None) == 1
