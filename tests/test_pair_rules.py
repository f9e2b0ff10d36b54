"""The pairing rules of the step-pair list walk (SVSA_ATTN_STEP_PAIRS), read
from the kernel source (runs without a GPU).

A step of the walk holds two union entries whose keep masks over the four
query sub-blocks of a workgroup are disjoint, so each sub-block still sees
each of its kept key blocks exactly once ([PSA] App. B, Alg. 2: every query
block attends to its own kept key blocks only).  The rule table must therefore
list only disjoint, non-empty mask pairs; it lists every such pair once
(4 bits: (3^4 - 2 * 2^4 + 1) / 2 = 25 unordered pairs), and fuller steps
(more keepers in the pair) come first.
"""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rules():
    src = open(os.path.join(ROOT, "block_sparse_attention_17_amd", "csrc", "attn.hip")).read()
    n = int(re.search(r"constexpr int kPairRules = (\d+);", src).group(1))
    body = re.search(r"kPairRule\[kPairRules\]\[2\] = \{(.*?)\};", src, re.S).group(1)
    body = re.sub(r"//[^\n]*", "", body)
    pairs = [(int(a), int(b)) for a, b in re.findall(r"\{\s*(\d+)\s*,\s*(\d+)\s*\}", body)]
    return n, pairs


def test_rule_table_is_every_disjoint_pair_once():
    n, pairs = _rules()
    assert n == len(pairs) == 25
    for a, b in pairs:
        assert 0 < a < 16 and 0 < b < 16, (a, b)
        assert a & b == 0, (a, b)
    unordered = {frozenset(p) for p in pairs}
    assert len(unordered) == 25
    every = {frozenset((a, b)) for a in range(1, 16) for b in range(1, 16) if a != b and a & b == 0}
    assert unordered == every


def test_rules_take_fuller_steps_first():
    _, pairs = _rules()
    filled = [bin(a | b).count("1") for a, b in pairs]
    assert filled == sorted(filled, reverse=True)
    # within equal fill: 3 + 1 before 2 + 2 (a bucket of three keepers has
    # only one partner mask), then 2 + 1, then 1 + 1
    sizes = [max(bin(a).count("1"), bin(b).count("1")) for a, b in pairs]
    assert sizes[:4] == [3] * 4 and sizes[4:7] == [2] * 3
