"""bench.py's host side without a GPU: the one-GPU rule, and the traffic
record it reads (profiles/traffic.json) against the kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_is_reported_only_for_its_kernel():
    """bench.py reports the committed counters while the kernel sources hash
    to the profiled version, and null once they changed."""
    import bench
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    if rec["kernel_source_sha256_16"] != bench.kernel_source_hash():
        for name in ("tp_share", "compute_heavy"):
            got, note = bench.measured_traffic(name)
            assert got is None and "changed" in note
        return
    import workloads as wl
    for name in wl.WORKLOADS:
        got, note = bench.measured_traffic(name)
        want = rec["workloads"][name]
        assert got == pytest.approx(want["hbm_bytes_per_launch"]), note
        # FETCH_SIZE and WRITE_SIZE (KiB per dispatch), scaled by the copy calibration
        scaled = (want["fetch_size_kib"] * rec["calibration"]["FETCH_SIZE"]["factor"]
                  + want["write_size_kib"] * rec["calibration"]["WRITE_SIZE"]["factor"]) * 1024
        assert got == pytest.approx(scaled, rel=1e-9)
        assert got >= want["algorithmic_bytes"]
        cf = bench.counter_figures(name)
        # the MFMA instruction count is the GEMM's own flop count, 2MNK
        assert cf["mfma_flops_per_launch_counters"] == wl.workload(name).flops
        assert 0.0 < cf["mfma_busy"] < 1.0
    assert bench.measured_traffic("no_such_workload")[0] is None


def test_algorithmic_work_of_the_named_workloads():
    """flops 2MNK; bytes A and B once, every peer once, C written once."""
    import workloads as wl
    for name in ("tp_share", "reduce_heavy", "compute_heavy", "wide_many_peer"):
        w = wl.workload(name)
        assert w.flops == 2 * w.M * w.N * w.K
        assert w.algorithmic_bytes == 2 * w.M * w.K + 2 * w.K * w.N + 4 * w.peers * w.M * w.N + 4 * w.M * w.N


class _FakeLib:
    """Stands in for the binding: launches are counted, and the launch with
    index `faulty` ends in a timeout that mk_get_stats reports (stickily)
    at the next call, as the library does."""

    def __init__(self, faulty):
        self.faulty = faulty
        self.launches = 0
        self.pending = 0

    def gemm_reduce_local(self, *a, **k):
        if self.launches == self.faulty:
            self.pending |= 1
        self.launches += 1

    def get_stats(self, maps=False, raise_on_error=True):
        bits, self.pending = self.pending, 0
        rc = -4 if bits else 0
        return {"rc": rc, "status": rc, "status_name": "MK_ERR_TIMEOUT" if bits else "MK_OK",
                "sticky_errors": bits}


class _Ev:
    def __init__(self, enable_timing=True):
        pass

    def record(self, stream):
        pass

    def elapsed_time(self, other):
        return 1.0


class _Torch:
    class cuda:
        Event = _Ev

        @staticmethod
        def synchronize():
            pass


@pytest.mark.parametrize("faulty", [0, 7, 19])
def test_a_failed_launch_anywhere_in_a_leg_fails_the_bench(faulty):
    """A timeout in any launch of a timed leg (first, middle, last) makes the
    leg's status check end the bench with a non-zero exit and no line."""
    import bench
    fake = _FakeLib(faulty)
    bench.time_leg(lambda: fake.gemm_reduce_local(), 20, 0, None, None, _Torch, settle_s=0)
    assert fake.launches == 20
    with pytest.raises(SystemExit) as e:
        bench.check_leg(fake, "fused")
    assert e.value.code == 3


def test_a_failed_launch_while_settling_fails_the_bench():
    """The untimed settling launches count too: the leg's status check covers
    every launch since the previous check."""
    import bench
    fake = _FakeLib(faulty=2)
    ms, _ = bench.time_leg(lambda: fake.gemm_reduce_local(), 5, 1, None, None, _Torch, settle_s=0.01)
    assert len(ms) == 5 and fake.launches >= 4 + 1 + 5
    with pytest.raises(SystemExit) as e:
        bench.check_leg(fake, "fused")
    assert e.value.code == 3


def test_settle_defaults_and_flag():
    import bench
    assert bench.parse([]).settle_ms == pytest.approx(bench.SETTLE_S * 1e3)
    assert bench.parse(["--settle-ms", "0"]).settle_ms == 0


def test_a_clean_leg_passes_the_status_check():
    import bench
    fake = _FakeLib(faulty=-1)
    fake.gemm_reduce_local()
    assert bench.check_leg(fake, "fused")["status"] == 0


def test_bench_defaults_to_the_largest_workload():
    import bench
    import workloads as wl
    args = bench.parse([])
    assert args.workload == "all" and bench.HEADLINE == "compute_heavy"
    biggest = max(wl.WORKLOADS.values(), key=lambda w: w.flops)
    assert biggest.name == bench.HEADLINE
    assert set(bench.SUITE) == set(wl.WORKLOADS)


def test_allgather_algorithmic_bytes():
    """AllGather+GEMM share: every shard read once and written once into the
    gathered A, B read once, C written once."""
    import bench
    import workloads as wl
    w = wl.ag_workload("ag_tp_share")
    R = w.peers + 1
    assert bench.ag_algorithmic_bytes(w) == (2 * R * w.M * w.K * 2 + 2 * w.K * w.N
                                            + 4 * R * w.M * w.N)
    assert set(bench.AG_SUITE) == set(wl.AG_WORKLOADS)


def test_ring_attention_algorithmic_work():
    """Ring Attention share: 4 S (R S) D H flops; Q, K, V read once, every
    arriving K and V read once and written once, O (fp32) and LSE written."""
    import bench
    import workloads as wl
    w = wl.ra_workload("ra_sp_share")
    e = w.S * w.H * w.D
    assert w.flops == 4 * w.S * (w.ranks * w.S) * w.D * w.H
    assert bench.ra_algorithmic_bytes(w) == 3 * 2 * e + (w.ranks - 1) * 2 * 2 * 2 * e + 4 * e + 4 * w.S * w.H
    assert set(bench.RA_SUITE) == set(wl.RA_WORKLOADS)
