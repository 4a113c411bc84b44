"""bench.py without a GPU: the multi-GPU request is refused with a message, and the rocprofv3
summarisers (kernel statistics, HBM traffic with the copy-probe scaling, MFMA counters) read
counter files of the layout rocprofv3 writes."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_kernel_summary(tmp_path):
    _write(str(tmp_path / "tr" / "t_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
           [["void moe::gemv::gate_up_kernel<1, 1, 64, 8>(int)", 10, 800000, 80000, 60.0, 78000, 83000],
            ["moe::combine_kernel<1, 64>(float)", 10, 50000, 5000, 4.0, 4000, 6000]])
    out = tmp_path / "k.md"
    bench.summarize_kernels(str(tmp_path / "tr"), str(out), "cmd")
    text = out.read_text()
    lines = [ln for ln in text.splitlines() if ln.startswith("| void") or ln.startswith("| moe")]
    assert lines[0].startswith("| void moe::gemv::gate_up_kernel<1, 1, 64, 8> | 10 | 80.00 |")  # largest total first
    assert "command: `cmd`" in text


def test_traffic_summary_scales_by_the_copy_probe(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    # the copy probe moved 512 MiB; FETCH_SIZE reports half of it (factor 2), WRITE_SIZE all of it
    probe = 512 << 20
    _write(str(tmp_path / "f" / "p_counter_collection.csv"), hdr,
           [["void at::native::neg_kernel(float)", "FETCH_SIZE", probe / 2 / 1024],
            ["void moe::gemv::gate_up_kernel<1, 1, 64, 8>(int)", "FETCH_SIZE", 1000.0],
            ["void moe::gemv::gate_up_kernel<1, 1, 64, 8>(int)", "FETCH_SIZE", 1200.0]])
    _write(str(tmp_path / "w" / "p_counter_collection.csv"), hdr,
           [["void at::native::neg_kernel(float)", "WRITE_SIZE", probe / 1024],
            ["void moe::gemv::gate_up_kernel<1, 1, 64, 8>(int)", "WRITE_SIZE", 10.0]])
    out = tmp_path / "t.md"
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "f", "w", "gemv", probe, 123.0)
    vals = dict(ln.split(": ", 1) for ln in out.read_text().splitlines() if ln.startswith(("traffic_bytes", "source_hash")))
    # mean fetch 1100 KiB x 2 + write 10 KiB x 1
    assert float(vals["traffic_bytes_per_launch"]) == (1100.0 * 2 + 10.0) * 1024
    assert vals["source_hash"] == bench.source_hash(bench.GATE_UP_SOURCES["gemv"])


def test_mfma_summary(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    k = "void moe::gemm::gemm_kernel<2, true>(int)"
    _write(str(tmp_path / "m" / "p_counter_collection.csv"), hdr,
           [[k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9], [k, "SQ_INSTS_VALU_MFMA_MOPS_F8", 0],
            [k, "GRBM_GUI_ACTIVE", 8 * 1e6], [k, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1024 * 1e6]])
    out = tmp_path / "m.md"
    bench.summarize_mfma(str(tmp_path / "m"), str(out), "cmd")
    row = [ln for ln in out.read_text().splitlines() if "gemm_kernel" in ln][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[4] == f"{1e9 * 512 / 1e12:.4f}"   # issued TFLOP: MOPS x 512 flops
    assert cells[6] == "0.250"                    # busy / (1024 SIMDs x active cycles per XCD)


def test_source_hash_ignores_comments_only():
    import tempfile
    d = tempfile.mkdtemp()
    a, b, c = (os.path.join(d, n) for n in ("a.h", "b.h", "c.h"))
    open(a, "w").write("int f(int x) { return x + 1; }  // one\n")
    open(b, "w").write("/* a comment */\nint f(int x) {\n  return x + 1;  // other\n}\n")
    open(c, "w").write("int f(int x) { return x + 2; }\n")
    h = lambda p: bench.source_hash([os.path.relpath(p, bench.ROOT)])
    assert h(a) == h(b) and h(a) != h(c)
