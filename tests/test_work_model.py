"""The benchmark's work model against the sizes the pages print
(tests/golden/page_numbers.json, each entry cited there)."""
import json
import os

import bench

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_attention_matrix_size():
    g = GOLD["attention_matrix_100_frames"]
    tokens = g["frames"] * g["tokens_per_frame"]
    assert tokens == g["total_tokens"]
    entries, fp16_bytes = bench.attention_matrix(tokens, 2)
    _, fp32_bytes = bench.attention_matrix(tokens, 4)
    assert abs(entries - g["entries"]) / g["entries"] < 0.005      # printed to 3 digits
    assert round(fp16_bytes / 1e9) == g["fp16_gigabytes"]
    assert round(fp32_bytes / 1e9) == g["fp32_gigabytes"]


def test_worked_example_patch_count():
    g = GOLD["worked_example_patches"]
    side = g["image_side"] // g["patch_side"]
    assert side * side == g["patches_per_frame"]
    assert g["frames"] * side * side == g["total_patches"]


def test_flop_model_consistency():
    # frame attention is global attention restricted to N diagonal blocks
    N, L, H = 100, 1374, 16
    assert bench.flops_frame(N, L, H) * N == bench.flops_global(N * L, H)
    # SGA with every token kept costs exactly global attention
    assert bench.flops_sga(N * L, N * L, H) == bench.flops_global(N * L, H)
    # gather reads K and V once and writes the kept rows of both (bf16)
    assert bench.bytes_gather(10, 4, 2) == 2 * 10 * 2 * 64 * 2 + 2 * 4 * 2 * 64 * 2


def test_sga_window_reduces_keys_by_stride_area():
    g = GOLD["sga_window"]
    # on a grid divisible by the stride, one kept patch per s x s window
    from tests.oracle_pins import kept_per_frame_closed_form
    gh = gw = 8
    assert kept_per_frame_closed_form(gh, gw, 0, g["stride"], g["stride"], 0, 0) * g["stride"] ** 2 \
        == gh * gw * g["kept_per_full_window"]


def test_cpu_baseline_weights_layers_by_count(monkeypatch):
    # the step time is each kind of layer's oracle time on the sampled rows,
    # weighted by how often the step runs it, scaled by rows of step / rows
    import oracle
    from vga_inputs import tiny_qkv

    clock = iter([0.0, 1.0, 10.0, 12.0])       # frame layer 1 s, SGA layer 2 s
    monkeypatch.setattr(bench.time, "perf_counter", lambda: next(clock))
    monkeypatch.setattr(oracle, "attention", lambda *a, **k: None)

    class F:  # the fields cpu_baseline reads
        num_frames, tokens_per_frame, grid_h, grid_w, num_heads = 2, 69, 8, 8, 2
        tokens = 138

    class P:
        stride_h = stride_w = 2
        phase_h = phase_w = 0
        diagonal, mean_fill = True, 1

    q, k, v = tiny_qkv(138, 2, 64, seed=0)
    res = bench.cpu_baseline("tiny", F, [P], ["frame"], (q, k, v), 23, counts=[2, 3])
    assert abs(res["seconds_per_step"] - (2 * 1.0 + 3 * 2.0) * 138 / 23) < 1e-9
    assert abs(res["value"] - 138 / res["seconds_per_step"]) < 1e-9
    assert "2xframe+3xsga" in res["sample"]


def test_projection_flops():
    # y = x W^T + b: one multiply-add per (token, input, output) feature
    assert bench.flops_linear(137400, 1024, 3072) == 2 * 137400 * 1024 * 3072
    # the QKV projection is three output projections' worth of work
    assert bench.flops_linear(7, 64, 192) == 3 * bench.flops_linear(7, 64, 64)


def test_bench_refuses_more_than_one_gpu():
    # the timed path runs on one device; more ranks stop before any GPU call
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
