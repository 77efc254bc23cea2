"""The rocprof harness's arithmetic on synthetic rocprofv3 output (no GPU):
kernel names, per-dispatch counter averages, the copy calibration of the HBM
counters, and the derived clock, MFMA and LDS utilisation."""
import csv
import os

import pytest

from block_masked_attention_amd import rocprof

K = "void bdattn::(anonymous namespace)::bwd_dq_kernel<true, 128>(bdattn::BwdArgs)"


def _write(d, name, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, f"run_{name}.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _counters(d, per_kernel):
    rows = []
    for i, (k, cs) in enumerate(per_kernel):
        grid = cs.pop("_grid", 131072)
        for disp in range(cs.pop("_dispatches", 1)):
            for c, v in cs.items():
                rows.append(dict(Dispatch_Id=f"{i}.{disp}", Kernel_Name=k, Grid_Size=grid,
                                 Counter_Name=c, Counter_Value=v))
    _write(d, "counter_collection", rows)


def test_short_names():
    assert rocprof.short_name(K) == "bwd_dq_kernel<true, 128>"
    assert rocprof.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    assert rocprof.short_name("bdattn::(anonymous namespace)::store_dq(float const*, "
                              "unsigned short*, unsigned short*, long, long, float)") == "store_dq"
    assert rocprof.short_name("void bdattn::(anonymous namespace)::fill_zero_f32(float*, long)") \
        == "fill_zero_f32"


def test_one_kernel_backward_profile(tmp_path):
    """--bwd fused10: the atomic requests of the write pass are reported per
    launch, the summaries get their own name, and the dominant kernel is
    reported in the dK/dV slot (where bench.py times it) under that name."""
    assert rocprof.profile_key("64k") == "64k"
    assert rocprof.profile_key("64k", 1, "fused10") == "64k_bwd_fused10"
    assert rocprof.profile_key("256k", 16, "fused10") == "256k_docs16_bwd_fused10"
    t = str(tmp_path)
    kf = "void bdattn::(anonymous namespace)::bwd_fused_kernel<true, 128, true>(bdattn::BwdArgs, float*)"
    kz = "bdattn::(anonymous namespace)::fill_zero_f32(float*, long)"
    _write(t + "/trace", "kernel_stats", [
        dict(Name=kf, Calls=1, AverageNs=4.0e8, MinNs=4.0e8, MaxNs=4.0e8, Percentage=90.0),
        dict(Name=kz, Calls=1, AverageNs=1.0e5, MinNs=1.0e5, MaxNs=1.0e5, Percentage=0.1)])
    _write(t + "/trace", "agent_info", [dict(Name="gfx950", Simd_Count=1024, Cu_Count=256,
                                             Num_Xcc=8)])
    _counters(t + "/fetch", [(rocprof.COPY_KERNEL, dict(FETCH_SIZE=524288)),
                             (kf, dict(FETCH_SIZE=1000.0)), (kz, dict(FETCH_SIZE=1.0))])
    _counters(t + "/write", [(rocprof.COPY_KERNEL, dict(WRITE_SIZE=1048576)),
                             (kf, dict(WRITE_SIZE=64.0, TCC_EA0_ATOMIC_sum=1024.0, _dispatches=2)),
                             (kz, dict(WRITE_SIZE=8.0, TCC_EA0_ATOMIC_sum=0.0))])
    for p in ("sq1", "sq2"):
        _counters(t + "/" + p, [(kf, dict(GRBM_GUI_ACTIVE=8 * 8.0e8))])
    args = [rocprof.counters(t + "/" + p) for p in ("fetch", "write", "sq1", "sq2")]
    s = rocprof.summarise(rocprof.durations(t + "/trace"), *args, rocprof.agent(t + "/trace"))
    r = s["kernels"]["bwd_fused_kernel<true, 128, true>"]
    assert r["atomic_requests"] == pytest.approx(1024.0)  # two dispatches of 1024: per launch
    assert s["kernels"]["fill_zero_f32"]["atomic_requests"] == 0.0
    assert "atomic requests" in rocprof.markdown(s, "64k_bwd_fused10", "cmd")
    dest = str(tmp_path / "profiles")
    rocprof.write_profiles(dest, "8k", "cmd", t + "/trace", *args, rocprof.agent(t + "/trace"), s,
                           bwd="fused10")
    txt = open(os.path.join(dest, "bdattn_8k_bwd_fused10_hbm_traffic.md")).read()
    assert "TCC_EA0_ATOMIC_sum" in txt and "BDATTN_BWD=fused10" in txt
    assert "kernel: bwd_dkdv" in txt and "workload: 8k_bwd_fused10" in txt


def test_summary_arithmetic(tmp_path):
    t = str(tmp_path)
    _write(t + "/trace", "kernel_stats", [dict(Name=K, Calls=2, AverageNs=2.0e6)])  # 2 ms
    _write(t + "/trace", "agent_info", [dict(Name="gfx950", Simd_Count=1024, Cu_Count=256,
                                             Num_Xcc=8)])
    # the copy reads 2^30 bytes but FETCH_SIZE reports half of it: scale 2
    _counters(t + "/fetch", [(rocprof.COPY_KERNEL, dict(FETCH_SIZE=524288)),
                             (K, dict(FETCH_SIZE=1000.0, _dispatches=2))])
    _counters(t + "/write", [(rocprof.COPY_KERNEL, dict(WRITE_SIZE=1048576)),
                             (K, dict(WRITE_SIZE=500.0))])
    cycles = 2.0e9 * 2.0e-3  # a 2 GHz clock over 2 ms
    _counters(t + "/sq1", [(K, dict(GRBM_GUI_ACTIVE=8 * cycles))])
    _counters(t + "/sq2", [(K, dict(GRBM_GUI_ACTIVE=8 * cycles,
                                    SQ_VALU_MFMA_BUSY_CYCLES=0.5 * 1024 * cycles,
                                    SQ_LDS_IDX_ACTIVE=0.25 * 256 * cycles,
                                    SQ_INSTS_MFMA=100.0, SQ_INSTS_VALU=300.0,
                                    SQ_INSTS_LDS=150.0, SQ_INSTS_SALU=50.0,
                                    SQ_LDS_BANK_CONFLICT=0.0))])
    s = rocprof.summarise(rocprof.durations(t + "/trace"), rocprof.counters(t + "/fetch"),
                          rocprof.counters(t + "/write"), rocprof.counters(t + "/sq1"),
                          rocprof.counters(t + "/sq2"), rocprof.agent(t + "/trace"))
    assert s["fetch_scale"] == pytest.approx(2.0) and s["write_scale"] == pytest.approx(1.0)
    r = s["kernels"]["bwd_dq_kernel<true, 128>"]
    assert r["ms"] == pytest.approx(2.0) and r["calls"] == 2
    # 1000 KiB per dispatch (2000 over two dispatches), times the scale 2
    assert r["hbm_read_gb"] == pytest.approx(1000 * 1024 * 2 / 1e9, abs=0.01)
    assert r["hbm_write_gb"] == pytest.approx(500 * 1024 / 1e9, abs=1e-3)
    assert r["clock_ghz"] == pytest.approx(2.0)
    assert r["mfma_busy"] == pytest.approx(0.5)
    assert r["lds_busy"] == pytest.approx(0.25)
    assert r["valu_per_mfma"] == pytest.approx(3.0) and r["lds_per_mfma"] == pytest.approx(1.5)
    md = rocprof.markdown(s, "256k", "python -m block_masked_attention_amd.rocprof")
    assert "| `bwd_dq_kernel<true, 128>` | 2 | 2 | 50% | 25% |" in md


def test_calibration_uses_the_large_copy_only(tmp_path):
    """The runtime also dispatches its copy kernel for small uploads; only
    the 1 GiB calibration copy (the largest grid) may set the scale factors."""
    t = str(tmp_path)
    _counters(t + "/fetch", [(rocprof.COPY_KERNEL, dict(FETCH_SIZE=8.0, _grid=1024, _dispatches=2)),
                             (rocprof.COPY_KERNEL, dict(FETCH_SIZE=524288.0)),
                             (K, dict(FETCH_SIZE=1000.0))])
    c = rocprof.counters(t + "/fetch")
    assert c[rocprof.COPY_KERNEL]["FETCH_SIZE"] == pytest.approx(524288.0)
    assert c[rocprof.COPY_KERNEL]["_dispatches"] == 1
    assert rocprof.lce_counters(t + "/fetch")[rocprof.COPY_KERNEL]["FETCH_SIZE"] == \
        pytest.approx(524288.0)


def test_repository_summaries(tmp_path):
    """The four summaries written from one run: every table present, and the
    machine-readable traffic lines name the longest main kernel, the current
    kernel source hash and its scaled HBM bytes per launch."""
    import re

    t = str(tmp_path)
    F = "void bdattn::(anonymous namespace)::fwd_kernel<true, 128, false>(bdattn::FwdArgs)"
    _write(t + "/trace", "kernel_stats", [
        dict(Name=K, Calls=1, AverageNs=3.0e6, MinNs=3.0e6, MaxNs=3.0e6, Percentage=60.0),
        dict(Name=F, Calls=1, AverageNs=2.0e6, MinNs=2.0e6, MaxNs=2.0e6, Percentage=40.0)])
    _write(t + "/trace", "agent_info", [dict(Name="gfx950", Simd_Count=1024, Cu_Count=256,
                                             Num_Xcc=8)])
    _counters(t + "/fetch", [(rocprof.COPY_KERNEL, dict(FETCH_SIZE=524288)),
                             (K, dict(FETCH_SIZE=1000.0)), (F, dict(FETCH_SIZE=10.0))])
    _counters(t + "/write", [(rocprof.COPY_KERNEL, dict(WRITE_SIZE=1048576)),
                             (K, dict(WRITE_SIZE=500.0)), (F, dict(WRITE_SIZE=5.0))])
    _counters(t + "/sq1", [(K, dict(GRBM_GUI_ACTIVE=1e7)), (F, dict(GRBM_GUI_ACTIVE=1e7))])
    _counters(t + "/sq2", [(K, dict(GRBM_GUI_ACTIVE=1e7, SQ_INSTS_MFMA=10.0, SQ_INSTS_VALU=30.0,
                                    SQ_INSTS_LDS=5.0, SQ_INSTS_SALU=1.0)),
                           (F, dict(GRBM_GUI_ACTIVE=1e7))])
    args = [rocprof.counters(t + "/" + p) for p in ("fetch", "write", "sq1", "sq2")]
    dev = rocprof.agent(t + "/trace")
    s = rocprof.summarise(rocprof.durations(t + "/trace"), *args, dev)
    dest = str(tmp_path / "profiles")
    rocprof.write_profiles(dest, "8k", "python -m block_masked_attention_amd.rocprof ...",
                           t + "/trace", *args, dev, s)
    for kind in ("rocprof_summary", "kernel_trace", "hbm_traffic", "sq_counters"):
        assert os.path.getsize(os.path.join(dest, f"bdattn_8k_{kind}.md")) > 200
    txt = open(os.path.join(dest, "bdattn_8k_hbm_traffic.md")).read()
    m = dict(re.findall(r"^(\w+):\s*(\S+)\s*$", txt, re.M))
    assert m["kernel"] == "bwd_dq" and m["workload"] == "8k"
    assert m["kernel_source"] == rocprof.kernel_source_hash()
    assert float(m["hbm_bytes_per_launch"]) == pytest.approx((1000 * 2 + 500) * 1024, rel=1e-3)
    # 1e7 GUI-active cycles over 8 XCDs in 3 ms: 0.4167 GHz
    assert float(m["clock_ghz"]) == pytest.approx(1e7 / 8 / 3e-3 / 1e9, abs=1e-3)
    sq = open(os.path.join(dest, "bdattn_8k_sq_counters.md")).read()
    assert "| derived: VALU instructions per MFMA | 3.00 |" in sq


def test_lce_roles_follow_the_transposes_in_the_kernel_names():
    """The linear cross-entropy's three library products are told apart by
    the transposes Tensile writes into their names; the row kernels by name."""
    from block_masked_attention_amd.rocprof import lce_role
    assert lce_role("Cijk_Alik_Bljk_BBS_BH_Bias_HAS_MT256x256x64_MI16x16x1") == "lce_logits"
    assert lce_role("Cijk_Ailk_Bljk_BBS_BH_MT256x256x64") == "lce_dh"
    assert lce_role("Cijk_Ailk_Bjlk_BSS_BH_MT256x256x64") == "lce_dw"
    assert lce_role("bdattn::(anonymous namespace)::lce_fused_kernel(float const*, int)") == "lce_rows"
    assert lce_role("__amd_rocclr_copyBuffer") is None
    assert lce_role("void at::native::vectorized_elementwise_kernel<4>") is None


def test_kernel_source_hash_ignores_comments(tmp_path):
    """A committed profile stays valid across comment edits of the kernel
    sources, not across code edits."""
    import shutil
    src = os.path.join(rocprof.ROOT, "block_masked_attention_amd", "csrc")
    for f in rocprof.KERNEL_SOURCES:
        shutil.copy(os.path.join(src, f), tmp_path / f)
    base = rocprof.kernel_source_hash(str(tmp_path))
    assert base == rocprof.kernel_source_hash()
    k = tmp_path / "kernels.hip"
    text = k.read_text()
    k.write_text("// a new comment line\n" + text.replace("\n", "  // trailing note\n", 1))
    assert rocprof.kernel_source_hash(str(tmp_path)) == base
    k.write_text(text.replace("kNegInf", "kNegInf ", 1) + "\nint unused_symbol;\n")
    assert rocprof.kernel_source_hash(str(tmp_path)) != base
