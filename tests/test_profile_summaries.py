"""The reduction of rocprofv3 output into the profiles/ tables (bench.py --summarize-profile), on
small synthetic CSV files written the way rocprofv3 writes them: kernel names are labelled,
dispatches are grouped by the marker ranges they ran in, counter readings are scaled by the
copy kernel's reading of a known size, and the traffic a bench line reports is the recorded one
only while the kernel sources are unchanged."""
import csv
import os
import statistics

import pytest

import bench

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")

DEC_BF16 = "void smla::(anonymous namespace)::decode_stage1_mfma<1, false, true, false>(smla::Stage1Args)"
DEC_FP8 = "void smla::(anonymous namespace)::decode_stage1_mfma<2, false, true, false>(smla::Stage1Args)"
UNION_BF16 = "void smla::(anonymous namespace)::decode_stage1_mfma<1, true, true, false>(smla::Stage1Args)"
COPY = ("void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, "
        "at::native::binary_internal::MulFunctor<float> >, std::array<char*, 2ul> >(int, ...)")


def _write_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_kernel_labels():
    assert bench.kernel_label(DEC_BF16) == "decode_stage1_mfma<bf16>"
    assert bench.kernel_label(DEC_FP8) == "decode_stage1_mfma<fp8>"
    assert bench.kernel_label(UNION_BF16) == "decode_stage1_mfma<bf16, union>"
    assert bench.kernel_label("void smla::(anonymous namespace)::decode_stage1_mfma<2, false, true, true>(x)") == \
        "decode_stage1_mfma<fp8>"
    assert bench.kernel_label("smla::decode_stage2_packed(smla::Stage2Args)") == "decode_stage2_packed"
    assert bench.kernel_label("smla::decode_stage2(smla::Stage2Args)") == "decode_stage2"
    assert bench.kernel_label("void smla::union_bitmap_kernel<16>(...)") == "union_bitmap_kernel<16>"
    assert bench.kernel_label("void smla::union_sort_kernel<4, 2>(...)") == "union_sort_kernel<4, 2>"
    assert bench.kernel_label("smla::resolve_kernel(...)") == "resolve_kernel"
    assert bench.kernel_label(COPY) is None
    assert bench.torch_label(COPY) == "torch vectorized_elementwise_kernel"


def test_trace_groups_dispatches_by_marker_range(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    d = tmp_path / "prof"
    d.mkdir()
    us = 1000                                          # timestamps in ns
    head = [26.0, 27.0, 26.5]
    kt = []
    t = 10 * us
    for v in head:                                     # three headline dispatches
        kt.append({"Kernel_Name": DEC_BF16, "Start_Timestamp": t, "End_Timestamp": t + int(v * us)})
        t += 40 * us
    kt.append({"Kernel_Name": COPY, "Start_Timestamp": 300 * us, "End_Timestamp": 310 * us})   # a flush: dropped
    kt.append({"Kernel_Name": DEC_FP8, "Start_Timestamp": 400 * us, "End_Timestamp": 446 * us})  # outside every form
    _write_csv(d / "run_kernel_trace.csv", kt)
    _write_csv(d / "run_marker_api_trace.csv", [
        {"Function": "workload: bf16 decode, batch 32", "Start_Timestamp": 0, "End_Timestamp": 200 * us},
        {"Function": "form: fused, back to back over rotating batches (the headline)", "Start_Timestamp": 5 * us,
         "End_Timestamp": 150 * us},
        {"Function": "workload: fp8 decode, batch 64", "Start_Timestamp": 350 * us, "End_Timestamp": 500 * us},
    ])
    bench.summarize_trace(str(d))
    text = (tmp_path / "decode_prefill_kernels_trace.md").read_text()
    rows = [ln for ln in text.splitlines() if ln.startswith("| decode_stage1_mfma")]
    assert len(rows) == 2
    cells = [c.strip() for c in rows[0].strip("|").split("|")]
    assert cells[:4] == ["decode_stage1_mfma<bf16>", "bf16 decode, batch 32",
                         "fused, back to back over rotating batches (the headline)", "3"]
    assert float(cells[4]) == pytest.approx(statistics.mean(head), abs=0.005)
    assert float(cells[6]) == pytest.approx(26.0) and float(cells[7]) == pytest.approx(27.0)
    cells = [c.strip() for c in rows[1].strip("|").split("|")]
    assert cells[:4] == ["decode_stage1_mfma<fp8>", "fp8 decode, batch 64", "set-up (outside the timed forms)", "1"]
    assert "vectorized_elementwise" not in text
    assert bench.sources_sha256(bench.ALL_KERNEL_SOURCES) in text


def _counter_rows(counter, readings):
    """rocprofv3 counter-collection rows: (kernel name, dispatch id, value, grid), several rows
    per dispatch adding up."""
    return [{"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
             "Counter_Value": val, "Start_Timestamp": 0, "End_Timestamp": 1000}
            for name, did, val, grid in readings]


def test_traffic_scaled_by_the_copy_reading(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    fd, wd = tmp_path / "fetch", tmp_path / "write"
    fd.mkdir()
    wd.mkdir()
    copy_grid = (64 << 20) // 4
    copy_kib = (256 << 20) / 1024
    # FETCH_SIZE reads the copy's 256 MiB as twice its size, WRITE_SIZE as its size
    _write_csv(fd / "run_counter_collection.csv", _counter_rows("FETCH_SIZE", [
        (COPY, 1, copy_kib, copy_grid), (COPY, 1, copy_kib, copy_grid),
        (DEC_BF16, 2, 60000.0, 256 * 512), (DEC_BF16, 2, 40000.0, 256 * 512),      # one dispatch: 100,000 KiB
        (DEC_BF16, 3, 80000.0, 256 * 512), (DEC_BF16, 3, 40000.0, 256 * 512),      # another: 120,000 KiB
        (COPY, 4, 5.0, 1024)]))                                                   # another torch kernel: ignored
    _write_csv(wd / "run_counter_collection.csv", _counter_rows("WRITE_SIZE", [
        (COPY, 1, copy_kib, copy_grid), (DEC_BF16, 2, 30000.0, 256 * 512), (DEC_BF16, 3, 34000.0, 256 * 512)]))
    with open(fd / "bench.json", "w") as fh:
        fh.write('[bench] log line\n{"algorithmic_bytes_step": 80264480, "fp8_kv_decode": {}}\n')
    bench.summarize_traffic(str(fd), str(wd))
    text = (tmp_path / "decode_kernels_hbm_traffic.md").read_text()
    rb = 110000.0 * 0.5 * 1024                          # mean FETCH_SIZE of the two dispatches, halved
    wb = 32000.0 * 1.0 * 1024
    line = next(ln for ln in text.splitlines() if ln.startswith("traffic_bytes_per_launch decode_stage1_mfma<bf16>"))
    tok = line.split()
    assert tok[2] == "bf16_batch_32"
    assert int(tok[3]) == round(rb + wb) and int(tok[5]) == round(rb) and int(tok[7]) == round(wb)
    row = next(ln for ln in text.splitlines() if ln.startswith("| decode_stage1_mfma<bf16>"))
    assert row.split("|")[-2].strip() == f"{(rb + wb) / 80264480:.3f}"
    assert "decode_stage1_mfma<fp8>" not in text       # no readings of it: no row

    # a bench run reports this traffic only while the kernel sources hash to the recorded value
    prof = tmp_path / "decode_kernels_hbm_traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.measured_traffic("decode_stage1_mfma<bf16>", "bf16_batch_32") == round(rb + wb)
    assert bench.measured_traffic("decode_stage1_mfma<bf16>", "fp8_batch_64") is None
    stale = text.replace(bench.sources_sha256(bench.KERNEL_SOURCES), "0" * 64)
    prof.write_text(stale)
    assert bench.measured_traffic("decode_stage1_mfma<bf16>", "bf16_batch_32") is None


def test_summarize_profile_rejects_wrong_arguments():
    with pytest.raises(SystemExit):
        bench.summarize_profile(["traffic", "only_one_dir"])
    with pytest.raises(SystemExit):
        bench.summarize_profile(["counters", "a"])


def test_committed_profiles_name_their_commands():
    """Every committed profile table gives the command that made it, and the sha256 of the
    sources it was taken on."""
    names = sorted(f for f in os.listdir(bench.PROFILE_DIR) if f.endswith(".md"))
    assert names
    for f in names:
        text = open(os.path.join(bench.PROFILE_DIR, f)).read()
        assert "```" in text and ("rocprofv3" in text or "bench.py" in text), f
        assert "sha256" in text, f
