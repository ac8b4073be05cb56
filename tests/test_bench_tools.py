"""bench.py's host-side tools, on the CPU:

- the clock sampler reads the amdgpu kernel driver's sysfs files correctly (a fake sysfs
  tree stands in for the card);
- the traffic record is computed correctly from rocprofv3 counter files
  (synthetic files stand in for a profiled run);
- `--shape` resolves to a workload of that size, and malformed shapes raise;
- `--gpus N` above 1 is refused with a message;
- the cache label says which timed calls fit the Infinity Cache.
"""
import os
import time

import pytest

import bench


def _card(root, sclk_text, power_uw=None, cap_uw=None, name="card0"):
    dev = os.path.join(root, name, "device")
    os.makedirs(os.path.join(dev, "hwmon", "hwmon0"))
    with open(os.path.join(dev, "pp_dpm_sclk"), "w") as f:
        f.write(sclk_text)
    if power_uw is not None:
        with open(os.path.join(dev, "hwmon", "hwmon0", "power1_input"), "w") as f:
            f.write(f"{power_uw}\n")
    if cap_uw is not None:
        with open(os.path.join(dev, "hwmon", "hwmon0", "power1_cap"), "w") as f:
            f.write(f"{cap_uw}\n")


def test_sampler_reads_marked_level_and_power(tmp_path):
    _card(str(tmp_path), "S: 1830Mhz *\n0: 500Mhz\n1: 2400Mhz\n", 1234500000, 1400000000)
    with bench.ClockSampler(period=0.001, root=str(tmp_path)) as c:
        time.sleep(0.02)
    s = c.summary()
    assert s["sclk_mhz_median"] == 1830 and s["sclk_mhz_min"] == 1830 and s["samples"] >= 1
    assert s["power_w_median"] == 1234.5 and s["power_cap_w"] == 1400.0
    assert s["sclk_top_level_mhz"] == 2400  # the highest numbered level, not the marked one


def test_sampler_marked_dpm_level(tmp_path):
    _card(str(tmp_path), "0: 500Mhz\n1: 2400Mhz *\n")
    with bench.ClockSampler(period=0.001, root=str(tmp_path)) as c:
        time.sleep(0.01)
    s = c.summary()
    assert s["sclk_mhz_median"] == 2400 and "power_w_median" not in s


def test_sampler_absent_or_ambiguous(tmp_path):
    with bench.ClockSampler(root=str(tmp_path / "none")) as c:
        pass
    assert c.summary() is None
    _card(str(tmp_path), "S: 1830Mhz *\n", name="card0")
    _card(str(tmp_path), "S: 1900Mhz *\n", name="card1")
    with bench.ClockSampler(root=str(tmp_path)) as c:
        pass
    assert c.summary() is None


# -- the HBM-traffic record written from rocprofv3 counter files ---------------

HEADER = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size",'
          '"Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count",'
          '"Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')
KERN = "void fa::(anonymous namespace)::flash_fwd_half<fa::BF16, 128, 8, 1, false, false>(fa::FwdParams)"
TORCH = "void at::native::elementwise_kernel<128, 4>(int, float)"
COPY = "__amd_rocclr_copyBuffer"
NAIVE = ["void fa::(anonymous namespace)::naive_scores_half<fa::BF16, 128>(fa::NaiveParams)",
         "void fa::(anonymous namespace)::naive_softmax<fa::BF16>(fa::NaiveParams)",
         "void fa::(anonymous namespace)::naive_pv_half<fa::BF16, 128>(fa::NaiveParams)"]


def _csv(path, counter, rows):
    with open(path, "w") as f:
        f.write(HEADER)
        for i, (name, grid, val) in enumerate(rows, 1):
            f.write(f'{i},{i},"Agent 1",1,1,1,{grid},1,"{name}",512,0,0,0,0,0,"{counter}",{val},0,1\n')
    return str(path)


def _copies(tmp_path):
    cf = _csv(tmp_path / "cf.csv", "FETCH_SIZE", [("elementwise", 1, 1.0), (COPY, 1, 512.0), (COPY, 1, 512.0)])
    cw = _csv(tmp_path / "cw.csv", "WRITE_SIZE", [(COPY, 1, 1024.0), (COPY, 1, 1024.0)])
    return cf, cw


def test_record_traffic(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    # a torch kernel (ignored), the warm-up call (left out), two timed calls
    f = _csv(tmp_path / "f.csv", "FETCH_SIZE", [(TORCH, 64, 7.0), (KERN, 1048576, 999.0), (KERN, 1048576, 100.0),
                                                 (KERN, 1048576, 300.0)])
    w = _csv(tmp_path / "w.csv", "WRITE_SIZE", [(TORCH, 64, 7.0), (KERN, 1048576, 5.0), (KERN, 1048576, 50.0),
                                                 (KERN, 1048576, 70.0)])
    cf, cw = _copies(tmp_path)
    rec = bench.record_traffic(f, w, cf, cw, copy_bytes=1 << 20)
    # copy of 1 MiB read as 512 KiB -> fetch scale 2; written as 1024 KiB -> scale 1
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_kib_per_launch"] == 200.0 and rec["write_kib_per_launch"] == 60.0
    assert rec["hbm_read_bytes_per_launch"] == 200 * 1024 * 2
    assert rec["hbm_write_bytes_per_launch"] == 60 * 1024
    assert rec["kernels"] == ["flash_fwd_half<BF16,128,8,1,false,false>"] and rec["dispatches_per_launch"] == 1
    assert rec["source_hash"] == bench.kernel_source_hash("flash")
    assert bench.measured_traffic("n32768_d128_bf16", "flash") == rec["hbm_bytes_per_launch"]


def test_record_traffic_sums_every_kernel_of_a_call(tmp_path, monkeypatch):
    """The three-pass path dispatches three kernels per call: the record sums
    all of them per call, after the warm-up call."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    vals = [[1000.0, 1000.0, 1000.0], [10.0, 20.0, 30.0], [30.0, 20.0, 10.0]]  # warm-up, then two calls
    f = _csv(tmp_path / "f.csv", "FETCH_SIZE", [(NAIVE[i], 8, v) for call in vals for i, v in enumerate(call)])
    w = _csv(tmp_path / "w.csv", "WRITE_SIZE", [(NAIVE[i], 8, 2 * v) for call in vals for i, v in enumerate(call)])
    cf, cw = _copies(tmp_path)
    rec = bench.record_traffic(f, w, cf, cw, workload="b32_n512_d64_bf16", entry="naive", copy_bytes=1 << 20)
    assert rec["dispatches_per_launch"] == 3 and len(rec["kernels"]) == 3
    assert rec["fetch_kib_per_launch"] == 60.0 and rec["write_kib_per_launch"] == 120.0
    assert rec["source_hash"] == bench.kernel_source_hash("naive")
    assert bench.measured_traffic("b32_n512_d64_bf16", "naive") == rec["hbm_bytes_per_launch"]


def test_record_traffic_rejects_uneven_dispatches(tmp_path, monkeypatch):
    import pytest

    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    f = _csv(tmp_path / "f.csv", "FETCH_SIZE", [(KERN, 1, 1.0)] * 4)
    cf, cw = _copies(tmp_path)
    with pytest.raises(ValueError):
        bench.record_traffic(f, f, cf, cw, copy_bytes=1 << 20)  # 4 dispatches are not 3 calls


def test_resolve_workload_shape_and_name():
    w = bench.resolve_workload("n32768_d128_bf16", None)
    assert (w.B, w.H, w.N, w.d, w.dtype) == (1, 16, 32768, 128, "bf16")
    w = bench.resolve_workload("n32768_d128_bf16", "2,8,4096,64,fp32")
    assert (w.name, w.B, w.H, w.N, w.d, w.dtype, w.seed, w.qk_sigma) == ("b2_h8_n4096_d64_fp32", 2, 8, 4096, 64,
                                                                            "fp32", 9, 1.0)
    for bad in ("1,8,4096,128", "1,8,4096,128,fp64", "0,8,4096,128,bf16", "1,8,x,128,bf16"):
        with pytest.raises(ValueError):
            bench.resolve_workload("n32768_d128_bf16", bad)


def _clock_record(start_ns, end_ns, pro_ns, loop_end_ns, hw, xcc, ghz=2.0, blk=0):
    tag = 1 | 4 << 8 | 1 << 16 | 128 << 24 | blk << 32
    return [start_ns // 10, end_ns // 10, int(pro_ns * ghz), int(loop_end_ns * ghz), int((end_ns - start_ns) * ghz),
            hw, xcc, tag]


def test_phase_clock_summary_synthetic():
    """Two CUs on two XCDs: CU A runs two 1000 ns workgroups with a 100 ns gap
    between them, CU B one 2100 ns workgroup; every workgroup spends 100 ns
    in its prologue; the cycle counts say 2 GHz."""
    cu_a, cu_b = 3 << 8, 5 << 8  # HW_ID CU_ID fields
    recs = (_clock_record(0, 1000, 100, 900, cu_a, 0, blk=0) + _clock_record(1100, 2100, 100, 900, cu_a, 0, blk=1)
            + _clock_record(0, 2100, 100, 2000, cu_b, 1, blk=2))
    s = bench.phase_clock_summary(recs, event_us=3.0)
    assert s["workgroups"] == 3 and s["cus"] == 2
    assert s["workgroups_per_cu"] == {1: 1, 2: 1}
    assert s["clock_ghz"] == pytest.approx(2.0)
    assert s["span_us"] == pytest.approx(2.1)
    assert s["prologue_us_min_median_max"] == [0.1, 0.1, 0.1]
    assert s["loop_us_min_median_max"] == [0.8, 0.8, 1.9]
    assert s["gap_end_to_next_start_us_median"] == pytest.approx(0.1)
    assert s["xcd_first_start_us"] == {0: 0.0, 1: 0.0}
    assert s["cu_last_end_us_min_median_max"] == [2.1, 2.1, 2.1]
    res, loop = s["share_with_k_resident"], s["share_with_k_in_loop"]
    assert sum(res.values()) == pytest.approx(1.0, abs=2e-3) and sum(loop.values()) == pytest.approx(1.0, abs=2e-3)
    # CU A is empty for 100 of its 2100 ns; B always holds one
    assert res[0] == pytest.approx(100 / 4200, abs=0.01) and res[1] == pytest.approx(4100 / 4200, abs=0.01)
    assert 2 not in res
    assert s["per_xcd"] == {0: {"clock_ghz": 2.0, "workgroups": 2, "last_end_us": 2.1},
                            1: {"clock_ghz": 2.0, "workgroups": 1, "last_end_us": 2.1}}


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n, monkeypatch, capsys):
    """The library has no multi-GPU path: `--gpus N` above 1 ends with exit
    status 2 and a message, before any GPU work."""
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", str(n)])
    assert bench.main() == 2
    assert "one GPU only" in capsys.readouterr().err


def test_cache_label():
    """The 4096- and 10,000-token and 512-token-batch calls fit the 256 MB
    Infinity Cache (warm across back-to-back calls); the 32K call does not."""
    from io_aware_tiled_06_amd.workloads import WORKLOADS

    assert bench.cache_label(WORKLOADS["n4096_d128_bf16"]).startswith("warm: Q, K, V, O and LSE (33.7 MB)")
    assert bench.cache_label(WORKLOADS["b32_n512_d64_bf16"]).startswith("warm")
    assert bench.cache_label(WORKLOADS["n32768_d128_bf16"]).startswith("cold: Q, K, V, O and LSE (539.0 MB)")
