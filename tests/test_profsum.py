"""The rocprofv3 summariser: the counter calibration takes the largest fill
and sum dispatches (the known 256 MiB write and read) even when smaller
kernels of the same name ran, and traffic per launch is scaled by it."""

import csv
import json
import os

from fp4_diffusion_transformer_amd import profsum

FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(d, name, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, name), "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_calibration_uses_the_largest_fill_and_sum(tmp_path, monkeypatch):
    mib = 256
    kib = (mib << 20) / 1024.0
    trace, fetch, write = (str(tmp_path / n) for n in ("trace", "fetch", "write"))
    os.makedirs(trace)
    with open(os.path.join(trace, "t_kernel_stats.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Name", "Calls", "AverageNs", "MinNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": "void fp4dit::gemm_fp4_kernel<2, 0, 3, 1>(GemmArgs)", "Calls": 3,
                    "AverageNs": 150000, "MinNs": 149000, "Percentage": 90})
    gemm = "void fp4dit::(anonymous namespace)::gemm_fp4_kernel<2, 0, 3, 1>(GemmArgs)"
    # FETCH_SIZE reports half the bytes, WRITE_SIZE all of them; a tiny fill
    # of an index buffer (FillFunctor<long>) comes first
    _write(fetch, "f_counter_collection.csv", [
        ("void at::native::reduce_kernel<512, 1>(float)", "FETCH_SIZE", kib / 2),
        (gemm, "FETCH_SIZE", 1000.0)])
    _write(write, "w_counter_collection.csv", [
        ("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<long> >", "WRITE_SIZE", 0.09),
        ("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >", "WRITE_SIZE", kib),
        (gemm, "WRITE_SIZE", 100.0)])
    out = str(tmp_path / "kernels_some_workload.txt")
    written = {}
    real_open = open

    def fake_open(path, mode="r", *a, **k):        # keep profiles/hbm_traffic.json untouched
        if str(path).endswith("hbm_traffic.json") and "w" in mode:
            class Sink:
                def __enter__(self):
                    return self

                def __exit__(self, *e):
                    return False

                def write(self, s):
                    written["json"] = written.get("json", "") + s
            return Sink()
        return real_open(path, mode, *a, **k)

    monkeypatch.setattr("builtins.open", fake_open)
    profsum.main(["profsum", trace, fetch, write, out, str(mib)])
    rec = json.loads(written["json"])["workloads"]["some_workload"]
    assert abs(rec["fetch_factor"] - 2.0) < 1e-12 and abs(rec["write_factor"] - 1.0) < 1e-12
    k = rec["kernels"]["gemm_swiglu<0,3,1>"]
    assert k["read_bytes"] == 1000.0 * 1024 * 2 and k["write_bytes"] == 100.0 * 1024
