"""CPU checks of bench.py's host logic: the one-GPU guard, the traffic record lookup and the
algorithmic work formulas."""
import importlib.util
import json
import os
import subprocess
import sys

from dispatch_expert_gemm_amd import workloads as WL
from dispatch_expert_gemm_amd.rocprof_summary import code_hash

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_code_hash_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f() { return 1; }  // one\n")
    b = tmp_path / "b.hip"
    b.write_text("// header\nint f()  {\n  return 1;   // other words\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f() { return 2; }\n")
    assert code_hash(str(a)) == code_hash(str(b)) != code_hash(str(c))


def test_traffic_record_lookup(tmp_path, monkeypatch):
    b = _bench()
    w = WL.WORKLOADS[2]
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "dispatch_expert_gemm_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "ffn.hip").write_text("int g() { return 0; }\n")
    rec = {"bytes_per_launch": 123, "kernel_prefix": "moe::ffn_gemm_bf16<2", "source": "ffn.hip",
           "source_code_sha256": code_hash(str(csrc / "ffn.hip"))}
    (tmp_path / "profiles" / f"hbm_traffic_ffn_gemm1_{w.name}.md").write_text(
        "# x\n\ntraffic-record: " + json.dumps(rec) + "\n")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.measured_traffic(w, "moe::ffn_gemm_bf16<2") == 123
    assert b.measured_traffic(w, "moe::ffn_gemm_f32<2") is None       # other kernel
    (csrc / "ffn.hip").write_text("int g() { return 1; }\n")           # code changed
    assert b.measured_traffic(w, "moe::ffn_gemm_bf16<2") is None
    assert b.measured_traffic(WL.WORKLOADS[4], "moe::ffn_gemm_bf16<2") is None   # no record


def test_headline_profiles_exist():
    # the kernel-duration and traffic summaries the bench line points to for its workload
    w = WL.WORKLOADS[4]
    for name in (f"kernel_stats_{w.name}.md", f"hbm_traffic_ffn_gemm1_{w.name}.md"):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        assert "ffn_gemm_bf16<2" in text and "Command:" in text


def test_route_source_defaults():
    b = _bench()
    # the correlated-routing workload keeps its planted logits; the others route from x
    assert [b.default_route_from(WL.WORKLOADS[i]) for i in range(1, 6)] == ["x"] * 4 + ["logits"]


def test_algorithmic_work_of_the_headline_workload():
    b = _bench()
    w = WL.WORKLOADS[2]
    a = b.algorithmic(w, w.N * w.k, 18634)
    # flops per launch 2 (N k + S N) H 2I for gate/up, half that for down
    assert a["gemm1_flops"] == 2 * (w.N * w.k + w.n_shared * w.N) * w.H * 2 * w.I
    assert a["gemm2_flops"] == a["gemm1_flops"] / 2
    # permute: unique x read once + every dispatched row written (bf16)
    assert a["permute_bytes"] == (w.N + w.N * w.k) * w.H * 2
    # weights of the 64 local experts and 2 shared experts, gate + up + down, read once
    assert a["gemm_weight_bytes"] == (64 + 2) * 3 * w.I * w.H * 2


def test_cpu_baseline_reports_stages_and_host():
    b = _bench()
    w = WL.WORKLOADS[1]
    host = dict(x=WL.gen_x(w), logits=WL.gen_logits(w), bias=WL.gen_bias(w),
                experts=WL.gen_experts(w, list(range(w.E)), 1), shared=WL.gen_shared_all(w))
    r = b.cpu_baseline(w, host, w.N)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
    assert set(r["stages_s"]) == {"route", "layout", "ffn", "combine"}
    assert 1 <= r["affinity"] <= r["cpu_count"]


def test_busy_summary_normalises_counters(tmp_path):
    from dispatch_expert_gemm_amd import rocprof_summary as R
    cols = ("Correlation_Id,Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,"
            "Start_Timestamp,End_Timestamp")
    lines = [cols]
    # two 500 us dispatches at 2.0 GHz on 8 XCDs, matrix cores busy 40% of 256 x 4 SIMD cycles
    for d in (1, 2):
        t0 = d * 10 ** 7
        cyc = 2.0e9 * 500e-6
        for name, v in (("GRBM_GUI_ACTIVE", 8 * cyc), ("SQ_VALU_MFMA_BUSY_CYCLES", 0.4 * cyc * 1024),
                        ("SQ_WAVES", 2048)):
            lines.append(f'{d},{d},"k",{name},{v},{t0},{t0 + 500000}')
    p = tmp_path / "c.csv"
    p.write_text("\n".join(lines) + "\n")
    row = R.busy(str(p), cus=256, xcds=8).splitlines()[2].split("|")
    assert [c.strip() for c in row[2:8]] == ["2", "500.0", "2.000", "40.0%", "0.00", "2048"]


def test_traffic_summary_scales_and_keeps_the_last_dispatches(tmp_path):
    from dispatch_expert_gemm_amd import rocprof_summary as R
    cols = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"

    def write(name, counter, copy_kib, vals):
        lines = [cols, f'1,"__amd_rocclr_copyBuffer",{counter},{copy_kib}']
        # two instances per dispatch (summed), dispatch ids after the copy
        for i, v in enumerate(vals):
            lines += [f'{i + 2},"void moe::ffn_gemm_bf16<2, 4>(x)",{counter},{v / 2}'] * 2
        (tmp_path / name).write_text("\n".join(lines) + "\n")
    # FETCH reads half the copy's bytes (scale 2); the first two launches are other launch kinds
    write("f.csv", "FETCH_SIZE", 512 * 1024, [10.0, 20.0, 1000.0, 1100.0])
    write("w.csv", "WRITE_SIZE", 1024 * 1024, [1.0, 2.0, 100.0, 120.0])
    src = tmp_path / "ffn.hip"
    src.write_text("int g() { return 0; }\n")
    out = R.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "moe::ffn_gemm_bf16<2",
                    "w", str(src), 1024, last=2)
    rec = json.loads(out.split("traffic-record: ")[1])
    assert rec["fetch_size_kib_raw"] == 1050.0 and rec["write_size_kib_raw"] == 110.0
    assert rec["bytes_per_launch"] == int((1050.0 * 2 + 110.0) * 1024)


def test_timeline_lists_one_step_with_early_side_work(tmp_path):
    from dispatch_expert_gemm_amd.rocprof_summary import timeline
    hdr = "Kind,Queue_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n"
    rows = [("A(x)", 1, 1000, 2000), ("S(y)", 2, 1500, 9000), ("A(x)", 1, 10000, 11000),
            ("B(z)", 1, 11000, 14000), ("S(y)", 2, 9500, 10500), ("A(x)", 1, 20000, 21000)]
    p = tmp_path / "t.csv"
    p.write_text(hdr + "".join(f"K,{q},\"{n}\",{b},{e}\n" for n, q, b, e in rows))
    text = timeline(str(p), "A", 1, before_us=1.0)
    lines = [l for l in text.splitlines() if l.startswith("| ") and "`" in l]
    # step 1 runs from 10000 to 20000 ns; the side dispatch at 9500 ns is within 1 us before it
    assert [l.split("`")[1] for l in lines] == ["S", "A", "B"]
    assert "| 2 | `S` | -0.5 | 0.5 | 1.0 |" in lines[0]
    assert "step 1: 4.0 us" in text and "next step starts at 10.0 us" in text
    try:
        timeline(str(p), "A", 2)
    except ValueError:
        pass
    else:
        raise AssertionError("a step past the last full one must be refused")
