"""Byte accounting of the measurement, pinned to figures printed on the pages.

The expected values are in tests/golden/page_examples.json, each with the page
and section it comes from.
"""
import json
import os

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "page_examples.json")


def _gold():
    with open(GOLDEN) as f:
        return json.load(f)


def test_kv_bytes_matches_page_product():
    for ex in _gold()["kv_bytes"]:
        got = synth.kv_bytes(ex["n_kv_head"], ex["head_dim"], ex["nkv"])
        assert got == ex["bytes"], ex["cite"]
        # the page rounds the product up to 4.3 MB; 4.19 MB is the exact value
        assert abs(got / 1e6 - ex["page_rounded_mb"]) < 0.15


def test_stream_rate_definition():
    """GB/s = K+V bytes / kernel time (R4 sections 1 and 2.4)."""
    for ex in _gold()["stream_rate"]:
        gbps = ex["bytes"] / (ex["us"] * 1e-6) / 1e9
        assert abs(gbps / ex["page_gbps"] - 1) <= ex["rel_tol"], (gbps, ex["cite"])


def test_red_lite_floor_bytes():
    for ex in _gold()["kv_elements"]:
        elems = ex["layers"] * synth.kv_bytes(ex["n_kv_head"], ex["head_dim"],
                                              ex["nkv"]) // 2
        assert abs(elems * 4 / 1e6 / ex["page_mb_at_4_bytes"] - 1) <= ex["rel_tol"]
        # the shape is the one the large-head workload uses
        assert (synth.CFG4.n_kv_head, synth.CFG4.head_dim, synth.CFG4_NKV,
                synth.CFG4_LAYERS) == (ex["n_kv_head"], ex["head_dim"], ex["nkv"],
                                       ex["layers"])
