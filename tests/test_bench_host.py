"""Host-side parts of the benchmark that need no GPU: the one-GPU guard,
the CPU oracle baseline record, and the algorithmic byte count the
roofline is priced on."""
import json
import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""  # no JSON line for a configuration that was not run


def test_cpu_baseline_record():
    rec = bench.cpu_baseline(synth.TINY, 16, False)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "routing of all 16 tokens" in rec["sample"]  # the sample says what was timed
    assert rec["cpu_model"] is not None and rec["blas"] and rec["host_cpus_visible"] >= 1


def test_counter_summary(tmp_path):
    """Gate+up bytes per launch from the two counter passes: per dispatch
    the counter summed over its rows, averaged over the gate+up dispatches
    only, scaled by the copy calibration, and stored with the source hash."""
    def rows(*r):
        return "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n" + "".join(
            f'{d},"void (anonymous namespace)::{k}(GemmArgs)",{c},{v}\n' for d, k, c, v in r)
    f = tmp_path / "f.csv"
    f.write_text(rows((1, "gemm_kernel<8, 4, 2, true>", "FETCH_SIZE", 100),
                      (1, "gemm_kernel<8, 4, 2, true>", "FETCH_SIZE", 20),
                      (2, "gemm_kernel<8, 4, 2, true>", "FETCH_SIZE", 140),
                      (3, "gemm_kernel<8, 8, 1, false>", "FETCH_SIZE", 9999)))
    w = tmp_path / "w.csv"
    w.write_text(rows((5, "gemv_kernel<true, true>", "WRITE_SIZE", 3),
                      (6, "gemv_kernel<false, true>", "WRITE_SIZE", 777)))
    out = tmp_path / "traffic.json"
    b = bench.summarize_counters("plateau:M=4096", str(f), str(w), str(out))
    assert b == round(130 * 1024 * bench.FETCH_FACTOR + 3 * 1024 * bench.WRITE_FACTOR)
    assert bench.stored_traffic("plateau", 4096, str(out)) == b
    # the `--only` form of the key is stored under the benchmark's name
    assert bench.summarize_counters("skew:512", str(f), str(w), str(out)) == b
    assert bench.stored_traffic("skew", 512, str(out)) == b
    assert set(json.load(open(out))["gate_up_bytes_per_launch"]) == {"plateau:M=4096", "skew:M=512"}
    with pytest.raises(SystemExit):
        bench.summarize_counters("plateau 4096", str(f), str(w), str(out))


@pytest.mark.parametrize("shape", [synth.TINY, synth.FULL])
def test_bytes_per_expert_closed_form(shape):
    """Codes are half a byte per weight and every 32 inputs of a row share
    one 2-byte scale: gate+up has 2I rows of H inputs, down H rows of I."""
    H, I = shape.H, shape.I
    w13, w2 = bench.bytes_per_expert(shape)
    assert w13 == 2 * I * H // 2 + 2 * (2 * I * H // 32)
    assert w2 == H * I // 2 + 2 * (H * I // 32)
    if shape is synth.FULL:  # the 384-expert layer's figures
        assert (w13, w2) == (16_515_072, 8_257_536)


def test_stored_traffic_only_for_the_current_sources(tmp_path):
    """The bench line's traffic figure is the stored counter reading for its
    workload and M, and null once the kernel sources differ from those the
    counters were taken on."""
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"source_sha256_16": bench.source_hash(),
                             "gate_up_bytes_per_launch": {"decode:M=9": 123}}))
    assert bench.stored_traffic("decode", 9, str(p)) == 123
    assert bench.stored_traffic("decode", 1, str(p)) is None
    assert bench.stored_traffic("plateau", 9, str(p)) is None
    p.write_text(json.dumps({"source_sha256_16": "0" * 16, "gate_up_bytes_per_launch": {"decode:M=9": 123}}))
    assert bench.stored_traffic("decode", 9, str(p)) is None
    p.write_text("not json")
    assert bench.stored_traffic("decode", 9, str(p)) is None
    assert bench.stored_traffic("decode", 9, str(tmp_path / "missing.json")) is None
