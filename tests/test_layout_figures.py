"""Closed-form pins of the entry-record and indexer-key sizes against the figures the pages
print (tests/golden/page_figures.json carries each figure with its citation)."""
import json
import os

import numpy as np

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def record_bytes(orc, D=512, R=64):
    nope, rope, scale = orc.quant_kv(np.ones((1, D), np.float32), R)
    return nope.nbytes + rope.nbytes + scale.nbytes


def key_bytes(orc, d=128):
    c, s = orc.quant_mxfp4(np.ones((1, d), np.float32))
    return c.nbytes + s.nbytes


def test_record_and_key_sizes(orc):
    assert record_bytes(orc) == 448 + 128 + 4
    assert key_bytes(orc) == 64 + 4


def test_kv_about_two_percent_of_gqa8(orc):
    sh = GOLD["model_shapes"]
    rec, key = record_bytes(orc), key_bytes(orc)
    csa = rec / sh["csa_ratio"] + key / sh["csa_ratio"]
    hca = rec / sh["hca_ratio"]
    layers = sh["layers_pro"]
    n_csa = (layers - 2) // 2            # first two layers HCA, then CSA/HCA alternate
    n_hca = layers - n_csa
    per_token = (n_csa * csa + n_hca * hca) / layers
    baseline = 2 * 8 * 128 * 2           # K and V, 8 KV heads, head dim 128, BF16
    frac = per_token / baseline
    assert abs(frac - GOLD["kv_fraction_vs_bf16_gqa8_hd128_at_1m"]["value"]) < 0.005


def test_split_precision_nearly_halves(orc):
    frac = (448 + 2 * 64) / (2 * 512)
    assert 0.45 < frac < 0.6 and abs(frac - GOLD["split_precision_kv_vs_all_bf16"]["value"]) < 0.1


def test_swa_about_eight_times_compressed(orc):
    rec = record_bytes(orc)
    uncompressed = 448 + 2 * 64          # one token in the split format, without a scale
    compressed = (rec / 4 + rec / 128) / 2
    assert abs(uncompressed / compressed - GOLD["swa_kv_vs_compressed_kv"]["value"]) < 0.5
