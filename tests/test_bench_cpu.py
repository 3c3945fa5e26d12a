"""Host logic of bench.py (no GPU): the rocprofv3 counter scaling that turns
FETCH_SIZE / WRITE_SIZE KiB into bytes per launch, the source-digest check
that keeps stale counter figures out of the JSON line, and the refusal of
runs on more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _counter_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, KiB); several rows may share a dispatch."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, name, v in rows:
            w.writerow([d, name, counter, v])


def test_traffic_from_scales_counters_by_the_copy(tmp_path):
    copy_bytes = 1 << 20
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    gemm = "void tpr::(anonymous namespace)::gemm_bf16_dma_kernel<false>(tpr::GemmBatch)"
    ce = "void tpr::(anonymous namespace)::ce_pair_kernel<0>(unsigned short const*)"
    # the copy reads 1 MiB: FETCH_SIZE shows 512 KiB (scale 2), WRITE_SIZE 1024 KiB (scale 1)
    _counter_csv(fetch, "FETCH_SIZE", [(1, "void at::native::neg_kernel_cuda(float)", 512.0),
                                       (2, gemm, 60.0), (2, gemm, 40.0), (3, gemm, 300.0), (4, ce, 50.0)])
    _counter_csv(write, "WRITE_SIZE", [(1, "void at::native::neg_kernel_cuda(float)", 1024.0),
                                       (2, gemm, 10.0), (3, gemm, 30.0), (4, ce, 5.0)])
    out_path = tmp_path / "traffic.json"
    out = bench.traffic_from(str(fetch), str(write), copy_bytes, out_path=str(out_path))
    assert out["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert out["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    assert out["FETCH_SIZE"]["gemm_bf16_dma_kernel"]["launches"] == 2  # rows of one dispatch are summed
    assert out["gemm_bf16_dma_kernel_bytes_per_launch"] == pytest.approx((100 + 300) / 2 * 1024 * 2 + 20 * 1024)
    assert out["ce_pair_kernel_bytes_per_launch"] == pytest.approx(50 * 1024 * 2 + 5 * 1024)
    on_disk = json.loads(out_path.read_text())
    assert on_disk["kernel_source_digest"] == bench.kernel_source_digest()
    assert on_disk == json.loads(json.dumps(out))


def test_traffic_from_needs_exactly_one_copy_dispatch(tmp_path):
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [(2, "gemm_bf16_dma_kernel", 1.0)])
    _counter_csv(write, "WRITE_SIZE", [(2, "gemm_bf16_dma_kernel", 1.0)])
    with pytest.raises(SystemExit):
        bench.traffic_from(str(fetch), str(write), 1 << 20, out_path=str(tmp_path / "t.json"))


def test_stored_traffic_only_for_the_current_sources(tmp_path):
    path = tmp_path / "traffic.json"
    key = "gemm_bf16_dma_kernel_bytes_per_launch"
    path.write_text(json.dumps({"kernel_source_digest": bench.kernel_source_digest(), key: 123.0}))
    assert bench.stored_traffic(key, path=str(path)) == 123.0
    assert bench.stored_traffic("other_kernel_bytes_per_launch", path=str(path)) is None
    path.write_text(json.dumps({"kernel_source_digest": "0" * 16, key: 123.0}))
    assert bench.stored_traffic(key, path=str(path)) is None
    assert bench.stored_traffic(key, path=str(tmp_path / "missing.json")) is None


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env=dict(os.environ, **env), timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
