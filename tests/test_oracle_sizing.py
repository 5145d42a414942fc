"""Pins of the oracle's closed forms against the numbers page 1 prints
(golden/page1_sizing.json holds each value with its place on the page)."""
import json
import os

import oracle

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page1_sizing.json")))
D, EB = G["kv_dim"], G["elem_bytes"]


def test_caps_printed():
    for c in G["caps"]:
        assert oracle.compressed_cap(c["ctx"], c["ratio"]) == c["cap"], c["cite"]


def test_per_layer_bytes_printed():
    for c in G["per_layer_bytes"]:
        b = oracle.pinned_bytes(c["ctx"], [c["ratio"]], D, EB)
        assert abs(b / c["unit"] - c["printed"]) <= c["half_ulp"], (c["cite"], b)


def test_group_bytes_printed():
    for c in G["group_bytes"]:
        layers = c["layers"] if isinstance(c["layers"], list) else [c["layers"]]
        ratios = []
        for r, n in zip(c["ratios"], layers):
            ratios += [r] * n
        b = oracle.pinned_bytes(c["ctx"], ratios, D, EB)
        assert abs(b / c["unit"] - c["printed"]) <= c["half_ulp"], (c["cite"], b)


def test_log_identities():
    for c in G["log_identities"]:
        if c["what"] == "max_capacity":
            assert oracle.max_capacity(c["window"], c["gpu_chunks"]) == c["value"]
        elif c["what"] == "gpu_chunks_total":
            assert c["layers"] * c["gpu_chunks"] == c["value"]
        elif c["what"] == "compressed_cap_total":
            assert c["layers"] * oracle.compressed_cap(c["ctx"], c["ratio"]) == c["value"]
        elif c["what"] == "pinned_mib":
            b = oracle.pinned_bytes(c["ctx"], [c["ratio"]] * c["layers"], D, EB)
            assert b == c["value"] * 2 ** 20


def test_swap_gpu_kv_printed():
    for c in G["swap_gpu_kv"]:
        b = c["layers"] * oracle.max_capacity(c["window"], c["gpu_chunks"]) * D * EB
        assert abs(b / c["unit"] - c["printed"]) <= c["half_ulp"], c["cite"]


def test_swap_toggle():
    for c in G["swap_toggle"]:
        cap = oracle.compressed_cap(c["ctx"], c["ratio"])
        assert oracle.swap_enabled(cap, c["gpu_chunks"]) == c["swap"], c["cite"]


def test_cap_closed_form_is_ceiling():
    # ceil(ctx / ratio) for every ctx in a range, against integer ceiling by brute force
    for ratio in (1, 3, 4, 128):
        for ctx in range(0, 600):
            n = 0
            while n * ratio < ctx:
                n += 1
            assert oracle.compressed_cap(ctx, ratio) == n
