"""Host-side rule of the decode-graph buckets (no GPU)."""
from paged_gqa_decode_head_amd.graphs import default_buckets


def test_default_buckets_follow_the_capture_rule():
    # every size up to 16, multiples of 8 above, and the maximum batch itself
    assert default_buckets(1) == [1]
    assert default_buckets(16) == list(range(1, 17))
    assert default_buckets(64) == list(range(1, 17)) + [24, 32, 40, 48, 56, 64]
    assert default_buckets(30) == list(range(1, 17)) + [24, 30]
