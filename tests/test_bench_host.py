"""Host-side arithmetic of the benchmark, on the CPU: the algorithmic byte and
flop counts the roofline fractions are quoted on (against hand sums for the
Mixtral-8x7B shape of the ExpertsInt8 latency table: hidden 4096,
intermediate 14336, 8 experts, top-2), the rate arithmetic, the counter
summary with its copy calibration, and the refusal of more than one GPU."""
import csv
import os
from types import SimpleNamespace

import numpy as np
import pytest

import bench


class _T:
    """A stand-in for a device tensor: element count and element size."""

    def __init__(self, n, size=1):
        self._n, self._s = n, size

    def numel(self):
        return self._n

    def element_size(self):
        return self._s


def _mixtral_int8_packed():
    E, K, N = 8, 4096, 14336
    return SimpleNamespace(w1=_T(E * 2 * N * K), s1=_T(E * 2 * N, 2), w2=_T(E * K * N), s2=_T(E * K, 2))


def test_moe_alg_counts_one_token_mixtral_int8():
    spec = SimpleNamespace(E=8, topk=2, K=4096, N=14336)
    ids = np.array([[3, 5]], np.int32)
    touched, g1, layer = bench.moe_alg_counts(spec, 1, ids, _mixtral_int8_packed())
    assert touched == 2
    # gate/up: 2 experts x (28672 x 4096 int8 codes + 28672 bf16 scales), x (4096 bf16), H (2 x 14336 bf16)
    assert g1["bytes"] == 2 * (28672 * 4096 + 28672 * 2) + 4096 * 2 + 2 * 14336 * 2 == 235061248
    assert g1["flops"] == 2 * 2 * 28672 * 4096
    # layer: both weight sets of the 2 experts, x read and the output row written (no H / Y round trips)
    w2 = 2 * (4096 * 14336 + 4096 * 2)
    assert layer["bytes"] == 2 * (28672 * 4096 + 28672 * 2) + w2 + 2 * 4096 * 2 == 352468992
    assert layer["flops"] == 2 * 2 * (28672 + 14336) * 4096 == 704643072


def test_moe_alg_counts_headline_batch_touches_every_expert():
    spec = SimpleNamespace(E=8, topk=2, K=4096, N=14336)
    ids = np.stack([np.arange(1024) % 8, (np.arange(1024) + 3) % 8], 1).astype(np.int32)
    touched, g1, layer = bench.moe_alg_counts(spec, 1024, ids, _mixtral_int8_packed())
    assert touched == 8
    assert g1["bytes"] == 8 * (28672 * 4096 + 28672 * 2) + 1024 * 4096 * 2 + 2048 * 14336 * 2 == 1007091712
    assert g1["flops"] == 2 * 2048 * 28672 * 4096 == 481036337152
    assert layer["flops"] == 6 * 2048 * 14336 * 4096 == 721554505728


def test_rates():
    r = bench.rates(8e9, 2.5e12, 1.0)  # 8 GB and 2.5 TFLOP in one millisecond
    assert r["GBps"] == pytest.approx(8000.0)
    assert r["frac_hbm"] == pytest.approx(1.0)
    assert r["TFLOPs"] == pytest.approx(2500.0)
    assert r["frac_mfma"] == pytest.approx(1.0)
    assert bench.rates(1, 5e12, 1.0, peak_tf=5000.0)["frac_mfma"] == pytest.approx(1.0)


def _write_counters(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(w.fieldnames, r)))


def test_summarize_counters_copy_calibration(tmp_path):
    """A 1 MiB calibration copy that counts 2048 KiB read and 1024 KiB written
    (a read counter at twice the bytes): a kernel's counts are scaled by 1/2 and
    1, averaged over its dispatches."""
    p = os.path.join(str(tmp_path), "p_counter_collection.csv")
    _write_counters(p, [
        ("__amd_rocclr_copyBuffer", 4096, 256, "FETCH_SIZE", 2048.0),
        ("__amd_rocclr_copyBuffer", 4096, 256, "WRITE_SIZE", 1024.0),
        ("__amd_rocclr_copyBuffer", 64, 64, "FETCH_SIZE", 3.0),  # a small runtime copy: not the calibration
        ("k", 1024, 256, "FETCH_SIZE", 100.0),
        ("k", 1024, 256, "FETCH_SIZE", 300.0),
        ("k", 1024, 256, "WRITE_SIZE", 10.0),
    ])
    rows = {(r["kernel"], r["grid"]): r for r in bench.summarize_counters([p], calib_bytes=1 << 20)}
    k = rows[("k", 1024)]
    assert k["FETCH_SIZE"] == pytest.approx(200.0) and k["FETCH_SIZE_dispatches"] == 2
    assert k["FETCH_SIZE_scale"] == pytest.approx(0.5)
    assert k["FETCH_SIZE_bytes"] == pytest.approx(200.0 * 1024 * 0.5)
    assert k["WRITE_SIZE_bytes"] == pytest.approx(10.0 * 1024)
    # without calibration only the raw means
    raw = {(r["kernel"], r["grid"]): r for r in bench.summarize_counters([p])}
    assert "FETCH_SIZE_bytes" not in raw[("k", 1024)]


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
