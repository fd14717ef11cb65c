"""The FLOP model used for throughput reporting, pinned to the pages' own FLOP accounting."""
import json
import os

import pytest

from axial_band_split_amd import roofline, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_flop_terms_match_printed_accounting():
    g = json.load(open(os.path.join(GOLDEN, "flop_terms.json")))
    w = synth.WORKLOADS["chunk8s_bf16"]                   # the vocals model at 801 frames
    s = roofline.shape_of(w, total_width=7916)
    f = roofline.flops_per_launch(s)
    L = w.depth
    # one "projection term" = one linear layer of one axis over all six layers, in MACs
    assert L * f["qkv"] / 2 / 1e9 == pytest.approx(g["projection_term_gmac"], abs=0.005)
    assert L * f["ffn1"] / 2 / 1e9 == pytest.approx(g["projection_term_gmac"], abs=0.005)
    assert L * f["attn_time"] / 2 / 1e9 == pytest.approx(g["attention_time_gmac"], abs=0.005)
    assert L * f["attn_band"] / 2 / 1e9 == pytest.approx(g["attention_freq_gmac"], abs=0.005)
    tot = roofline.flops_forward(s)
    assert tot["trunk"] / 2 / 1e9 == pytest.approx(g["trunk_gmac"], abs=0.05)
    # the printed per-chunk total leaves out the band split
    assert (tot["trunk"] + tot["mask"]) / 1e12 == pytest.approx(g["chunk_tflop"], abs=0.0005)
