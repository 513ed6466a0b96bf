"""Host logic of bench.py that needs no GPU: the kernel-source hash that ties a
committed profile to the code it measured, the counter summary's scaling of
rocprofv3 FETCH_SIZE / WRITE_SIZE by the device copy (checked by hand on a
synthetic pair of counter passes), and the one-GPU rule."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_code_only_drops_comments_and_keeps_literals():
    src = ('int a = 1;  // trailing\n/* block\n   comment */ const char* s = "x // y /* z */";\n'
           "char q = '\"';\tint b =\n  2; // \"quoted\" in a comment\n")
    assert bench._code_only(src) == 'int a = 1; const char* s = "x // y /* z */"; char q = \'"\'; int b = 2;'


def test_escaped_quote_inside_a_literal():
    assert bench._code_only('f("a\\"b // c"); // d') == 'f("a\\"b // c");'


@pytest.fixture
def source_copy(tmp_path, monkeypatch):
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_hash_ignores_comment_edits_but_not_code_edits(source_copy):
    before = bench.kernel_source_hash()
    rel = bench.KERNEL_SOURCES[0]
    path = source_copy / rel
    text = path.read_text(encoding="utf-8")
    path.write_text("// an added comment line\n" + text.replace("\n", "\n\n", 3), encoding="utf-8")
    assert bench.kernel_source_hash() == before
    path.write_text(text + "\nstatic int added_symbol = 1;\n", encoding="utf-8")
    assert bench.kernel_source_hash() != before


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write_counter_csv(path, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow([i, kernel, counter, value])


def test_counter_summary_scales_by_the_device_copy_and_reads_back(tmp_path, monkeypatch):
    # A synthetic pair of counter passes: the 2 GiB device copy reads as 1 GiB fetched and 2 GiB written
    # (factors 2 and 1, as on the device), two decode dispatches, one append + check, one merge.
    assert bench.COPY_BYTES == 2 * 1024 ** 3
    copy = "__amd_rocclr_copyBuffer"
    dec = "void fp8kv::(anonymous namespace)::decode_kernel<0, 128, 16, true>(fp8kv::DecodeParams)"
    app = "void fp8kv::(anonymous namespace)::append_check_kernel<0>(fp8kv::AppendParams, fp8kv::DecodeParams, long)"
    mrg = "void fp8kv::(anonymous namespace)::merge_kernel<128, 1>(fp8kv::DecodeParams)"
    out = tmp_path / "run"
    _write_counter_csv(str(out / "pmc_fetch_conc32" / "run_counter_collection.csv"),
                       [(copy, "FETCH_SIZE", 1048576), (dec, "FETCH_SIZE", 1000), (dec, "FETCH_SIZE", 1200),
                        (app, "FETCH_SIZE", 5), (mrg, "FETCH_SIZE", 20)])
    _write_counter_csv(str(out / "pmc_write_conc32" / "run_counter_collection.csv"),
                       [(copy, "WRITE_SIZE", 2097152), (dec, "WRITE_SIZE", 10), (dec, "WRITE_SIZE", 10),
                        (app, "WRITE_SIZE", 3), (mrg, "WRITE_SIZE", 4)])
    (out / "pmc_fetch_conc32" / "line.json").write_text(
        '{"legs": {"fp8": {"alg_bytes_decode": 2000000, "alg_bytes_step": 2100000}}}')
    written = {}
    monkeypatch.setattr(bench, "counters_path",
                        lambda wl, kv: written.setdefault((wl, kv), str(tmp_path / f"{wl}_{kv}.txt")))
    bench.summarize_workload_counters(str(out), "conc32")
    assert list(written) == [("conc32", "fp8")]          # no BF16 leg in the line: no BF16 summary
    vals = {}
    for ln in open(written[("conc32", "fp8")]):
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            vals[k.strip()] = v.strip()
    assert float(vals["fetch_scale"]) == 2.0 and float(vals["write_scale"]) == 1.0
    dec_bytes = 1100 * 1024 * 2 + 10 * 1024             # mean FETCH x 2 + mean WRITE x 1
    step_bytes = dec_bytes + (5 * 1024 * 2 + 3 * 1024) + (20 * 1024 * 2 + 4 * 1024)
    assert int(vals["decode_traffic_bytes_per_launch"]) == dec_bytes
    assert int(vals["step_traffic_bytes"]) == step_bytes
    assert float(vals["decode_traffic_over_algorithmic"]) == pytest.approx(dec_bytes / 2000000, abs=1e-4)
    assert float(vals["step_traffic_over_algorithmic"]) == pytest.approx(step_bytes / 2100000, abs=1e-4)
    # the bench reads the traffic back only while the summary's source hash is the current one
    assert bench.read_traffic("conc32", "fp8") == dec_bytes
    path = written[("conc32", "fp8")]
    text = open(path).read().replace(bench.kernel_source_hash(), "0000000000000000")
    open(path, "w").write(text)
    assert bench.read_traffic("conc32", "fp8") is None
