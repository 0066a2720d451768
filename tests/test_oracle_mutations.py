"""Every planted mistake in the oracle is caught by at least one pin.

Each ORC_MUTATE value in oracle/gqa_oracle.c plants one plausible mistake
(a wrong KV-head index, a dropped scale, a flipped RoPE sign, a strict `own`
comparison, an off-by-one window, a scaled sink, a strict `seen`, a swapped
page index, a wrong inv_freq denominator, truncating rounding, an ignored
cache row, reversed in-page offsets, a transposed Linear weight, a dropped
backward term, an unrounded default scale, an fp64 inv_freq pipeline). The oracle is
rebuilt with each one into a temporary directory; the pins must reject it.
"""
import os

import pytest

import oracle
from oracle import build as obuild
from tests import oracle_pins

MUTATIONS = {
    1: "kv head h % KvHeads instead of floor(h / G)",
    2: "softmax scale dropped",
    3: "rope sign flipped in the low half",
    4: "own mask strict (<) on positions",
    5: "window keeps W + 1 keys",
    6: "sink multiplied by the scale",
    7: "decode seen strict (<)",
    8: "paged page/offset swapped",
    9: "inv_freq uses D/2 in the exponent",
    10: "rounding truncates",
    11: "chunked prefill ignores the token's cache row",
    12: "paged chunk reverses offsets inside a page",
    13: "linear reads the weight transposed",
    14: "attention backward drops the softmax row term delta",
    15: "default scale left in fp64 (not rounded to f32)",
    16: "inv_freq evaluated in plain fp64, rounded to f32 only at the end",
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, mutation):
    lib = obuild.build(str(tmp_path / f"liboracle_m{mutation}.so"), mutation=mutation)
    o = oracle.Oracle(lib)
    assert o.mutation() == mutation
    bad = oracle_pins.failing_pins(o)
    assert bad, f"mutation {mutation} ({MUTATIONS[mutation]}) passed every pin"
