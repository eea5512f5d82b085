"""The shared-gate GPU tests cover each launch mode of the kernel: the token
counts they use (64, 1100 and 8200 for the edge cases, 1024 against 1100 and
8000 against 8200 for the bit-for-bit agreement) fall on both sides of the
two token thresholds in the kernel source."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _threshold(name):
    src = open(os.path.join(ROOT, "score_function_top_amd", "csrc", "router_gate.hip")).read()
    m = re.search(r"constexpr int64_t %s = (\d+);" % name, src)
    assert m, name
    return int(m.group(1))


def test_token_counts_straddle_the_mode_thresholds():
    split_max = _threshold("kGateSplitMaxTokens")   # one wave per half up to here
    late_min = _threshold("kGateLateMinTokens")     # routed half last from here
    assert split_max < late_min
    # edge cases: one token count per mode
    assert 64 <= split_max < 1100 < late_min <= 8200
    # agreement pairs: each pair crosses one threshold
    assert 1024 <= split_max < 1100
    assert 8000 < late_min <= 8200
