"""Host logic of the benchmark: the HBM traffic it reports comes from the committed PMC
profiles only while the kernel sources still hash to what the profile records, and is
summed from the profile's own table.  Synthetic profiles stand in for the committed ones,
so these checks do not depend on when the kernels were last profiled."""
import hashlib
import os

import bench


def _sha16(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(bench.ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def _prefill_profile(sha):
    return (f"kernel sources: prefill sha256[:16] {sha}, decode sha256[:16] 0000000000000000\n\n"
            "| kernel | workload | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | written GB |\n"
            "|---|---|---|---|---|---|\n"
            "| prefill_image_kernel<8> | global prefill T32768 | 1 | 1 | 3.790 | 0.537 |\n"
            "| prefill_band_kernel<8> | sliding prefill B4xT8192 | 1 | 1 | 1.000 | 0.540 |\n")


def _backward_profile(sha):
    return (f"kernel source: backward sha256[:16] {sha}\n\n"
            "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB (scaled) | written GB | algorithmic read / written GB |\n"
            "|---|---|---|---|---|---|\n"
            "| bwd_krot_kernel | 1 | 1 | 0.034 | 0.034 | x |\n"
            "| bwd_dq_kernel | 1 | 1 | 2.183 | 1.083 | x |\n"
            "| bwd_dkdv_kernel<4> | 1 | 1 | 1.635 | 0.168 | x |\n")


def test_prefill_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    p = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "_TRAFFIC_PROFILE", str(p))
    assert bench.profiled_traffic("global prefill T32768") is None          # no profile
    p.write_text(_prefill_profile(_sha16(bench._PREFILL_SOURCES)))
    assert abs(bench.profiled_traffic("global prefill T32768") - 4.327e9) < 1.0
    assert abs(bench.profiled_traffic("sliding prefill B4xT8192") - 1.54e9) < 1.0
    assert bench.profiled_traffic("no such workload") is None
    p.write_text(_prefill_profile("0123456789abcdef"))                      # sources changed since
    assert bench.profiled_traffic("global prefill T32768") is None


def test_backward_traffic_sums_the_call_and_follows_the_source_hash(tmp_path, monkeypatch):
    p = tmp_path / "backward.md"
    monkeypatch.setattr(bench, "_BACKWARD_PROFILE", str(p))
    assert bench.profiled_backward_traffic() is None
    p.write_text(_backward_profile(_sha16(bench._BACKWARD_SOURCES)))
    assert abs(bench.profiled_backward_traffic() - 5.137e9) < 1.0
    p.write_text(_backward_profile("0123456789abcdef"))
    assert bench.profiled_backward_traffic() is None
