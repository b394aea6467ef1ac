"""Host-side logic of bench.py, on the CPU: steps per graph, the byte counts
the roofline divides by, the dominant-kernel choice and the lookup of the
counter-based traffic figure."""
import bench


def test_steps_per_graph_divides_the_timed_steps():
    for steps in range(1, 200):
        d = bench.steps_per_graph(steps)
        assert 1 <= d <= bench.STEPS_PER_GRAPH and steps % d == 0
        assert all(steps % e for e in range(d + 1, bench.STEPS_PER_GRAPH + 1))
    assert bench.steps_per_graph(20) == 5 and bench.steps_per_graph(200) == 8 and bench.steps_per_graph(7) == 7


def test_algorithmic_bytes_hand_values():
    # q_proj, one token: x 8 KiB, A 128 KiB, h 64 B
    assert bench.shrink_bytes(1, 4096, 16) == 8192 + 131072 + 64
    # h 64 B, B 128 KiB, y read and written 16 KiB
    assert bench.expand_bytes(1, 16, 4096) == 64 + 131072 + 16384
    # plus eight fp32 workspace slices of 16 values
    assert bench.combine_bytes(1, 16, 4096, 8) == 512 + 64 + 131072 + 16384


def test_roofline_picks_the_kernel_with_the_most_time():
    fused = (10.0, 2, 4.0e6, "k_fused (M=1/16)", None)
    combine = (12.0, 2, 3.0e6, bench.COMBINE_KERNEL + " (M=64/256)", {"64": 5.0, "256": 7.0})
    r = bench.pick_roofline([fused, combine], lambda name: 123.0 if name.startswith(bench.COMBINE_KERNEL) else None)
    assert r["kernel"].startswith(bench.COMBINE_KERNEL) and r["traffic"] == 123.0
    assert r["avg_launch_us"] == 6.0 and r["algorithmic_bytes_per_launch"] == 1.5e6
    assert r["achieved"] == 250.0 and r["frac"] == round(250.0 / bench.HBM_PEAK_GBS, 4)
    # the single-launch candidate (per-M times None) unpacks the same way
    r = bench.pick_roofline([(20.0, 2, 4.0e6, "k_fused (M=1/16)", None), combine], lambda name: None)
    assert r["kernel"] == "k_fused (M=1/16)" and r["launch_us_per_m"] is None and r["traffic"] is None
    assert r["achieved"] == 200.0


def test_recorded_traffic_needs_the_current_kernel_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    f.write_text("source_hash: %s\nhbm_bytes M=1: 100\nhbm_bytes M=16: 300\n" % bench.kernel_source_hash())
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic(bench.COMBINE_KERNEL, [1, 16]) == 200.0
    assert bench.recorded_traffic(bench.COMBINE_KERNEL, [1, 16, 64]) is None        # M not recorded
    f.write_text("source_hash: 0000000000000000\nhbm_bytes M=1: 100\nhbm_bytes M=16: 300\n")
    assert bench.recorded_traffic(bench.COMBINE_KERNEL, [1, 16]) is None            # sources changed
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic(bench.COMBINE_KERNEL, [1]) is None

