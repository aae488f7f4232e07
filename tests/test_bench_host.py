"""Host-side pieces of bench.py (no GPU): the HBM traffic figure is reported only for the
kernel source and the workload run its counters were taken on."""
import json
import os

import bench


def test_traffic_only_for_its_workload_and_kernel():
    path = os.path.join(bench.ROOT, "profiles", "attn_bf16_wan_mixed_traffic.json")
    with open(path) as f:
        rec = json.load(f)
    khash = rec["kernel_hash"]
    assert bench.traffic_from_profiles(khash, rec["workload"]) == rec["bytes_per_launch"]
    assert bench.traffic_from_profiles(khash, "stripe_route") is None
    assert bench.traffic_from_profiles(khash, None) is None
    assert bench.traffic_from_profiles("0" * 16, rec["workload"]) is None

