"""Layout facts the pages print (tests/golden/layout.json), checked against the
generator constants and the oracle's index use."""
import json
from pathlib import Path

import numpy as np

import oracle
from mhc_inputs import HC, MIX

G = json.loads((Path(__file__).parent / "golden" / "layout.json").read_text())


def test_constants():
    assert HC == G["hc"]["value"] and MIX == G["mix"]["value"]
    for k, v in G["mix_hc"]["value"].items():
        hc = int(k)
        assert (2 + hc) * hc == v == hc + hc + hc * hc
    for tokens, nbytes in G["mix_scratch_bytes_90_sites"]["value"].items():
        assert int(tokens) * MIX * 4 * 90 == nbytes


def test_oracle_reads_the_printed_slices():
    # Put a distinct logit in each slot (scale 0, base = slot id) and read back where it lands.
    base = np.arange(MIX, dtype=np.float32) * 0.01
    pre, post, L = oracle.mix_activation(np.zeros((1, MIX)), np.ones(1), np.zeros(3, np.float32), base, 0.0, 1.0)
    s = G["slices"]["value"]
    sig = lambda z: 1 / (1 + np.exp(-z))
    assert np.allclose(pre[0], sig(base[s["pre"][0]:s["pre"][1]].astype(np.float64)))
    assert np.allclose(post[0], sig(base[s["post"][0]:s["post"][1]].astype(np.float64)))
    assert np.array_equal(L[0].ravel(), base[s["comb"][0]:s["comb"][1]].astype(np.float64))


def test_scale_order():
    assert G["scale_order"]["value"] == ["pre", "post", "comb"]
    d = np.zeros((1, MIX))
    d[0, 0] = d[0, 4] = d[0, 8] = 1.0
    pre, post, L = oracle.mix_activation(d, np.ones(1), np.array([1.0, 2.0, 3.0], np.float32),
                                         np.zeros(MIX, np.float32), 0.0, 1.0)
    sig = lambda z: 1 / (1 + np.exp(-z))
    assert np.isclose(pre[0, 0], sig(1.0)) and np.isclose(post[0, 0], sig(2.0)) and L[0, 0, 0] == 3.0
