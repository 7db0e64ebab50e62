"""Hand-derived fixtures (tests/golden/hand_cases.json) against the oracle."""
import json
import os

import numpy as np

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def test_nibble_bytes():
    for c in GOLD["nibble_bytes"]["cases"]:
        codes = np.array([c["codes"]])
        packed = oracle.pack_nibbles(codes)
        assert packed[0].tolist() == c["bytes"]
        back = oracle.unpack_nibbles(packed, signed=not c.get("unsigned", False))
        assert back[0].tolist() == c["codes"]


def test_activation_ties():
    for c in GOLD["activation_ties"]["cases"]:
        q, s, rs, _ = oracle.quant_act(np.array([c["row"]]), c["bits"])
        assert float(s[0]) == c["scale"]
        assert q[0].tolist() == c["codes"]
        assert rs[0] == sum(c["codes"])


def test_weight_asym():
    for c in GOLD["weight_asym"]["cases"]:
        codes, s, z, _, _ = oracle.quant_weights_asym(np.array([c["row"]]))
        assert float(s[0]) == c["scale"] and int(z[0]) == c["zp"]
        assert codes[0].tolist() == c["codes"]


def test_hadamard_4():
    h = GOLD["hadamard_4"]
    assert oracle.rotate(np.array([h["x"]]), 4)[0].tolist() == h["rotated"]
