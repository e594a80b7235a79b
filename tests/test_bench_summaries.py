"""bench.py's summaries of rocprofv3 output, on small synthetic CSVs in the
profiler's formats (no GPU): the byte-counter summary scales by the copy
kernel's counts and maps the pass's fixed launch order onto the decode
chain's ops; the kernel-trace summary finds the timed region right before
the launch-floor graph; the traffic lookup refuses a stale source hash."""
import csv
import json
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

PMC_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
            "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_pmc(path, counter, dispatches):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(PMC_COLS)
        for i, (name, grid, blk, val) in enumerate(dispatches):
            w.writerow([i + 1, i + 1, "Agent 1", 1, 1, 1, grid, 7, name, blk, 0, 0, 8, 0, 16, counter, val, 0, 1])


def pass_dispatches(fetch: bool):
    """The --pmc-pass order: 3 copies of 1 GiB, 2 steps of the 28-layer chain,
    3 one-launch batch-256 chains, 3 batch-1 chains, then one large shape;
    a torch kernel and a cos/sin table build interleaved (both ignored)."""
    kib = 1 << 20  # 1 GiB in KiB
    out = [("void kcr::copy_kernel(kcr::CopyArgs)", 67108864, 64, kib / 2 if fetch else kib)] * 3
    out.append(("void at::native::some_torch_kernel()", 1024, 256, 5.0))
    out.append(("void kcr::rope_table_kernel(kcr::TableArgs)", 1024, 256, 5.0))
    ops = [("void kcr::row_norm_wave_kernel<kcr::Bf16, 3, true>(kcr::NormArgs)", 16384, 64, 1600.0, 3200.0),
           ("void kcr::rope_token_kernel<kcr::Bf16, 8, false, 128, true>(kcr::RopeArgs)", 32768, 128, 1100.0, 2200.0),
           ("void kcr::row_norm_wave_kernel<kcr::Bf16, 3, true>(kcr::NormArgs)", 16384, 64, 1600.0, 3200.0),
           ("void kcr::swiglu_rows_kernel<kcr::Bf16, kcr::SiluMul>(kcr::SwigluRowArgs)", 327680, 256, 9000.0, 9000.0)]
    for _ in range(2 * 28):
        for n, g, b, fv, wv in ops:
            out.append((n, g, b, fv / 2 if fetch else wv / 2))
    out += [("void kcr::decode_chain_kernel<kcr::Bf16, 3, 512>(kcr::ChainArgs)", 131072, 512, 1.0)] * 3
    out += [("void kcr::decode_chain_kernel<kcr::Bf16, 3, 512>(kcr::ChainArgs)", 512, 512, 1.0)] * 3
    out += [("void kcr::swiglu_kernel<kcr::Bf16>(kcr::SwigluArgs)", 9175040, 64, 2.0)] * (5 if fetch else 7)
    return out


def test_counter_summary(tmp_path, capsys):
    fd, wd = str(tmp_path / "fetch"), str(tmp_path / "write")
    write_pmc(fd, "FETCH_SIZE", pass_dispatches(True))
    write_pmc(wd, "WRITE_SIZE", pass_dispatches(False))
    bench.counter_summary(fd, wd)
    text = capsys.readouterr().out
    block = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    assert block["scale_fetch"] == pytest.approx(2.0) and block["scale_write"] == pytest.approx(1.0)
    chain = block["decode_chain"]
    # FETCH counted half the bytes (scale 2), WRITE exactly: 1600 KiB read + 1600 KiB written
    assert chain["add_rmsnorm"]["traffic_bytes_per_launch"] == 1024 * (1600 + 1600)
    assert chain["add_rmsnorm"]["dispatches"] == 112 and chain["rope_kvstore"]["dispatches"] == 56
    assert chain["swiglu"]["traffic_bytes_per_launch"] == 1024 * (9000 + 4500)
    assert chain["one_launch_b256"]["grid"] == 131072 and chain["one_launch_b1"]["grid"] == 512
    assert chain["add_rmsnorm"]["source_sha256"] == bench.kernel_source_sha("add_rmsnorm")
    assert "some_torch_kernel" not in text and "rope_table_kernel" not in text


def test_counter_lookup_refuses_stale_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    entry = dict(traffic_bytes_per_launch=123, source_sha256="0" * 64)
    (prof / "hbm_bytes_counters.md").write_text("x\n```json\n" + json.dumps({"decode_chain": {"swiglu": entry}})
                                                 + "\n```\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda op: "1" * 64)
    traffic, note = bench.counter_traffic("swiglu")
    assert traffic is None and "changed" in note
    monkeypatch.setattr(bench, "kernel_source_sha", lambda op: "0" * 64)
    assert bench.counter_traffic("swiglu") == (123, None)


def test_trace_summary_timed_region(tmp_path, capsys):
    cols = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
            "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z",
            "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    kinds = [("void kcr::row_norm_wave_kernel<kcr::Bf16, 3, true>(kcr::NormArgs)", 16384, 64, 2000),
             ("void kcr::rope_token_kernel<kcr::Bf16, 8, false, 128, true>(kcr::RopeArgs)", 32768, 128, 3000),
             ("void kcr::row_norm_wave_kernel<kcr::Bf16, 3, true>(kcr::NormArgs)", 16384, 64, 2000),
             ("void kcr::swiglu_rows_kernel<kcr::Bf16, kcr::SiluMul>(kcr::SwigluRowArgs)", 327680, 256, 4000)]
    rows, t = [], 0
    steps = 3
    for k in range(112 * (steps + 2)):           # warm-up replays, then the timed ones
        n, g, b, dur = kinds[k % 4]
        rows.append((n, g, b, t, t + dur))
        t += dur + 1000
    for _ in range(112):                          # the launch-floor graph: 16-byte copies
        rows.append(("kcr::copy_kernel(kcr::CopyArgs)", 64, 64, t, t + 500))
        t += 1500
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "bench_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for i, (n, g, b, s, e) in enumerate(rows):
            w.writerow(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, i + 1, 3, n, i + 1, s, e, 0, 0, 8, 0, 16,
                        b, 1, 1, g, 1, 1])
    bench.trace_summary(str(d), steps)
    text = capsys.readouterr().out
    timed = text.split("## The timed region")[1]
    assert f"| {56 * steps} | 56 | 2.00 |" in timed.replace("`", "")
    assert f"| {28 * steps} | 28 | 4.00 |" in timed.replace("`", "")


def test_kernel_coverage_summary(tmp_path):
    """tests/kernel_coverage.py: compiled variants from nm's launch-stub
    symbols, run variants from a kernel trace (return type, parameter list and
    spacing ignored), and the variants that never ran listed by name."""
    import kernel_coverage as kc
    nm = ("0000000000001000 T kcr::__device_stub__copy_kernel(kcr::CopyArgs)\n"
          "0000000000002000 T void kcr::__device_stub__row_norm_kernel<kcr::Bf16, kcr::NormCfg<1, 3, 2, true, "
          "true, 1, false>, true, true>(kcr::NormArgs)\n"
          "0000000000003000 T void kcr::__device_stub__row_norm_kernel<kcr::F32, kcr::NormCfg<5, 2, 4, true, "
          "true, 1, false>, false, true>(kcr::NormArgs)\n"
          "0000000000004000 T kcr::run_norm(kcr::NormArgs const&, void*)\n")
    compiled = kc.compiled_kernels(nm)
    assert len(compiled) == 3
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "t_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Kernel_Name"])
        w.writerow(["KERNEL_DISPATCH", "kcr::copy_kernel(kcr::CopyArgs)"])
        w.writerow(["KERNEL_DISPATCH", "void kcr::row_norm_kernel<kcr::Bf16, kcr::NormCfg<1, 3, 2, true, true, 1, "
                                       "false>, true, true>(kcr::NormArgs)"])
        w.writerow(["KERNEL_DISPATCH", "void at::native::vectorized_elementwise_kernel<4>(int)"])
    ran = kc.traced_kernels(str(d))
    text = kc.summary(compiled, ran)
    assert "| `kcr::row_norm_kernel` | 2 | 1 |" in text
    assert "| all | 3 | 2 |" in text
    assert "kcr::row_norm_kernel<kcr::F32,kcr::NormCfg<5,2,4,true,true,1,false>,false,true>" in text
    assert "Every compiled" not in text


def test_source_hash_ignores_comments_only():
    """The counter summary's source hash changes with the code, not with its
    comments or layout; string literals that look like comments are code."""
    base = 'int f(int x) {  // doubles x\n    return 2 * x; /* the\n product */ }\nconst char* s = "a // b";\n'
    same = '/* header */\nint f(int x) {\n  return 2 * x;\n}\nconst char* s = "a // b";  // tail\n'
    assert bench.code_only(base) == bench.code_only(same)
    assert bench.code_only(base) != bench.code_only(base.replace("2 * x", "3 * x"))
    assert bench.code_only(base) != bench.code_only(base.replace('"a // b"', '"a // c"'))


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus above 1 (or a WORLD_SIZE above 1)
    exits with status 2 and says why, before touching a device."""
    import subprocess
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2, r.stderr
        assert "one GPU only" in r.stderr
        assert r.stdout == ""


def test_chain_roofline_picks_the_op_with_most_time(monkeypatch):
    """The roofline object names the chain op with the largest kernel time
    per step (per-launch time in a graph x launches per step), whichever op
    moves the most bytes, and its rate is its bytes per launch over that
    time."""
    import types
    import torch
    chain = types.SimpleNamespace(h=torch.zeros((256, 1536), dtype=torch.bfloat16), hidden=1536, inter=8960,
                                  hq=12, hkv=2, dh=128, positions=torch.full((256,), 4096, dtype=torch.int64))
    monkeypatch.setattr(bench, "counter_traffic", lambda op: (None, None))
    per_op = dict(add_rmsnorm=[4e-3] * 56 * 2, rope_kvstore=[4e-3] * 28 * 2, swiglu=[4e-3] * 28 * 2)
    copy_us = dict(add_rmsnorm=2.3, rope_kvstore=2.2, swiglu=4.0)
    nbytes = bench.chain_op_bytes(chain)
    # add_rmsnorm: 56 x 2.7 us = 151 us per step; SwiGLU moves 4x the bytes but 28 x 3.8 = 106 us
    graph = dict(add_rmsnorm=2.7, add_rmsnorm_2=2.7, rope_kvstore=2.6, swiglu=3.8)
    roof = bench.chain_roofline(chain, graph, per_op, 2, copy_us)
    assert roof["kernel"] == "add_rmsnorm"
    assert roof["launches_per_step"] == 56
    assert roof["achieved"] == pytest.approx(nbytes["add_rmsnorm"] / 2.7e-6 / 1e9, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 8000.0, rel=1e-3)
    assert sum(o["share_of_kernel_time"] for o in roof["chain_ops"].values()) == pytest.approx(1.0, abs=1e-3)
    # a slower SwiGLU takes the object over
    graph["swiglu"] = 6.0
    assert bench.chain_roofline(chain, graph, per_op, 2, copy_us)["kernel"] == "swiglu"
