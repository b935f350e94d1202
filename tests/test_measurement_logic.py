"""Host logic of the measurement path, on the CPU: kernel labels and profiler-name matching, the
traffic summary's scaling by the copy kernel, the bench's use of a committed traffic figure only for
the sources and kernel it was taken on, and the bench's parity check of the timed output."""
import csv
import importlib.util
import json
import os

import numpy as np
import pytest

import synthetic_inputs as si
from oracle import oracle as orc
from software_pipelined_tiled_amd import profsum

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def plan(**kw):
    p = dict(bm=256, bn=256, bk=64, stages=5, waves=8, mfma=16, persistent=1, group_m=8, load_path=1, grid=256,
             lds_bytes=163840, splits=1, stream=0)
    p.update(kw)
    return p


@pytest.mark.parametrize("p,label", [
    (plan(), "gemm_pp_kernel<256,256,64,5,waves=8,bf16,bf16>"),
    (plan(mfma=32), "gemm_pp_kernel<256,256,64,5,waves=8,bf16,bf16,mfma32x32x16>"),
    (plan(splits=2), "gemm_pp_kernel<256,256,64,5,waves=8,bf16,f32,splits=2>"),
    (plan(bm=128, bn=128, stages=4, waves=4, load_path=3), "gemm_dma_kernel<128,128,64,4,waves=4,bf16,bf16,staged>"),
    (plan(bm=32, bn=32, bk=128, stages=8, waves=2, stream=2), "gemm_dma_kernel<32,32,128,8,waves=2,bf16,bf16,stream=B>"),
    (plan(bm=32, bn=32, bk=128, stages=8, waves=2, stream=1), "gemm_dma_kernel<32,32,128,8,waves=2,bf16,bf16,stream=A>"),
    (plan(bm=128, bn=128, stages=2, waves=4, load_path=2), "gemm_reg_kernel<128,128,64,2,waves=4,bf16,bf16>"),
])
def test_kernel_label(p, label):
    assert profsum.kernel_label(p, "bf16", "bf16") == label


def test_kernel_name_matching():
    pp = plan()
    assert profsum.kernel_matches(pp, "void spt::gemm_pp_kernel<5, 16, __bf16, 1>(spt::GemmArgs)")
    assert profsum.kernel_matches(pp, "_ZN3spt14gemm_pp_kernelILi5ELi16EDF16_Li0EEEvNS_8GemmArgsE")  # left mangled
    assert not profsum.kernel_matches(pp, "_ZN3spt14gemm_pp_kernelILi5ELi32EDF16_Li0EEEvNS_8GemmArgsE")  # MFMA 32
    assert not profsum.kernel_matches(pp, "void spt::gemm_pp_kernel<2, 16, __bf16, 1>(spt::GemmArgs)")  # two stages
    d = plan(bm=32, bn=32, bk=128, stages=8, waves=2, stream=2)
    assert profsum.kernel_matches(d, "_ZN3spt15gemm_dma_kernelILi32ELi32ELi128ELi8ELi2ELi1EDF16_Li0ELi2EEEvNS_8GemmArgsE")
    assert not profsum.kernel_matches(d, "_ZN3spt15gemm_dma_kernelILi64ELi64ELi128ELi4ELi2ELi2EDF16_Li0ELi0EEEvNS_8GemmArgsE")
    # the reduction and staging kernels count toward a run, the probes do not
    plans = [d]
    assert profsum._run_kernel(plans, "void spt::splitk_reduce_kernel<0>(spt::ReduceArgs)")
    assert profsum._run_kernel(plans, "spt::stage_kernel(spt::StageArgs)")
    assert not profsum._run_kernel(plans, "(anonymous namespace)::copy16_kernel(unsigned int __vector(4) const*, ...)")


def test_plan_parts():
    single = {"plan": plan()}
    assert profsum.plan_parts(single) == [plan()]
    cut = {"plan": plan(load_path=3), "parts": {"dim": 1, "at": 4096, "first": plan(), "second": plan(bm=128)}}
    assert profsum.plan_parts(cut) == [plan(), plan(bm=128)]
    assert profsum.plan_parts({"plan": plan(), "parts": {"dim": -1, "at": 0, "first": plan()}}) == [plan()]


def write_counters(path, counter, gemm_kib, copy_kib, kernel):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        d = 0
        for v in copy_kib:
            d += 1
            w.writerow({"Dispatch_Id": d, "Kernel_Name": "(anonymous namespace)::copy16_kernel(...)",
                        "Counter_Name": counter, "Counter_Value": v})
        for v in gemm_kib:
            d += 1
            w.writerow({"Dispatch_Id": d, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_scales_by_the_copy_kernel_and_skips_the_cold_run(tmp_path):
    # four runs of one mainloop dispatch; the first (cold) run is left out of the mean. The copy kernel
    # moves 2^30 bytes each way: FETCH_SIZE reads half of that (scale 2), WRITE_SIZE all of it (scale 1)
    kernel = "_ZN3spt15gemm_dma_kernelILi32ELi32ELi128ELi8ELi2ELi1EDF16_Li0ELi2EEEvNS_8GemmArgsE"
    p = plan(bm=32, bn=32, bk=128, stages=8, waves=2, stream=2)
    write_counters(tmp_path / "f.csv", "FETCH_SIZE", [999999.0, 100.0, 110.0, 120.0], [524288.0], kernel)
    write_counters(tmp_path / "w.csv", "WRITE_SIZE", [77777.0, 8.0, 8.0, 8.0], [1048576.0], kernel)
    line = {"steps": 3, "warmup": 1, "extra": {"gemm_runs": 4},
            "config": {"workload": "c5_skinny_ragged_f16", "kernel": "k", "plan": p, "M": 32, "N": 8192, "K": 8192,
                       "out_dtype": "f16"}}
    (tmp_path / "b.json").write_text("noise\n" + json.dumps(line) + "\n")
    profsum.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "b.json"),
                    str(tmp_path / "out.json"), command="cmd")
    d = json.loads((tmp_path / "out.json").read_text())
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert d["read_bytes_per_launch"] == pytest.approx(110.0 * 1024 * 2.0)
    assert d["write_bytes_per_launch"] == pytest.approx(8.0 * 1024)
    assert d["gemm_dispatches_averaged"] == [3, 3]
    assert d["compulsory_bytes"] == (32 * 8192 + 8192 * 8192) * 2 + 32 * 8192 * 2
    assert d["kernel_source_sha"] == profsum.kernel_source_hash() and d["command"] == "cmd"


def test_bench_uses_traffic_only_for_its_sources_and_kernel(tmp_path, monkeypatch):
    bench = load_bench()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    good = {"kernel": "gemm_pp_kernel<256,256,64,5,waves=8,bf16,bf16>", "kernel_source_sha": profsum.kernel_source_hash(),
            "hbm_bytes_per_launch": 1.5e9}
    path = tmp_path / "profiles" / "traffic_c3_8192_bf16_bf16_0.json"
    path.write_text(json.dumps(good))
    assert bench.load_traffic("c3_8192_bf16_bf16", 0, good["kernel"]) == 1.5e9
    assert bench.load_traffic("c3_8192_bf16_bf16", 0, "gemm_pp_kernel<256,256,64,2,waves=8,bf16,bf16>") is None
    assert bench.load_traffic("c3_8192_bf16_bf16", 0, good["kernel"], cold=True) is None  # no _cold_b file
    assert bench.load_traffic("c3_8192_bf16_bf16", 1, good["kernel"]) is None
    path.write_text(json.dumps(dict(good, kernel_source_sha="0000000000000000")))
    assert bench.load_traffic("c3_8192_bf16_bf16", 0, good["kernel"]) is None


def test_bench_parity_checks_every_row_it_computes():
    # the timed output is compared with every oracle row the baseline computes: the oracle's own
    # result passes everywhere; one output moved far off is the one failure, and its index is reported
    bench = load_bench()
    M, N, K = 48, 40, 96
    a = si.make_matrix(M, K, si.F16, "uniform", 0xBE1)
    b = si.make_matrix(N, K, si.F16, "uniform", 0xBE2)
    c_ref, _, _ = orc.gemm(a, b, K, si.F16, si.F16)
    base, par = bench.cpu_baseline(a, b, K, si.F16, si.F16, c_ref.copy(), seconds=5.0, full_seconds=30.0)
    assert par["ok"] and par["n_checked"] == M * N and par["n_fail"] == 0 and par["max_err_over_tol"] == 0.0
    assert base["kind"] == "oracle" and base["cores"] >= 1 and base["value"] > 0
    bad = c_ref.copy()
    bad[37, 11] = si.to_f16_bits(np.array([1000.0], np.float32))[0]
    _, par = bench.cpu_baseline(a, b, K, si.F16, si.F16, bad, seconds=5.0, full_seconds=30.0)
    assert not par["ok"] and par["n_fail"] == 1 and par["worst_index"] == [37, 11]


def test_abtest_arguments_and_revision_label(tmp_path):
    from software_pipelined_tiled_amd import abtest
    with pytest.raises(SystemExit):
        abtest.main(["run", "x/libsptgemm.so", "--workloads", "c3,c9"])  # unknown workload, nothing run
    lib = tmp_path / "libsptgemm.so"
    lib.write_bytes(b"")
    assert abtest._revision(str(lib)) == "tree"
    (tmp_path / "REVISION").write_text("0123456789abcdef0123\n")
    assert abtest._revision(str(lib)) == "0123456789ab"
    # every timed workload is one whose shape the bit-exact checks cover with the same plan family
    assert {(m, n, k) for m, n, k, _ in abtest.WORKLOADS.values()} <= {(m, n, k) for m, n, k, _, _ in abtest.CHECKS}


def test_timeline_instruments_the_current_kernel():
    # the timeline tool's source transform still finds its anchors in the kernel as it stands: one
    # recorder, and a timestamp after each of the eight barriers of the phase stream
    from software_pipelined_tiled_amd import timeline
    src = open(os.path.join(ROOT, "software_pipelined_tiled_amd", "csrc", "spt_gemm_pp.hip")).read()
    out = timeline.instrument(src)
    assert out.count("barrier_sync(); rec();") == 8 and out.count("rec();") == 9
    assert "spt_timeline_read" in out and src.count("rec()") == 0
    with pytest.raises(ValueError):
        timeline.instrument(src.replace("barrier_sync();", "", 1))
