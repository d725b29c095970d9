"""Host logic of bench.py (no GPU): measurement windows, workload tags, the
one-GPU contract."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("R,L,at_least,want", [(1, 16, 64, 64), (3, 16, 64, 96), (21, 32, 128, 672), (5, 16, 16, 80),
                                               (1, 8, 1, 8)])
def test_cycle_steps_are_whole_cycles_of_every_pool(R, L, at_least, want):
    s = bench.cycle_steps(R, L, at_least)
    assert s == want
    assert s % (R * L) == 0 and s >= at_least


def test_workload_tags():
    from workloads import CONFIGS
    assert bench.extra_cfg("2") == CONFIGS[2]
    g = bench.extra_cfg("g128")
    assert (g.batch, g.num_slots, g.H_v, g.H_k, g.d, g.state_dtype) == (128, 128, 32, 16, 128, "f32")
    k = bench.extra_cfg("k256")
    base4 = CONFIGS[4]
    assert (k.batch, k.num_slots, k.H_v, k.H_k, k.d, k.decay, k.update, k.L) == (
        256, 256, base4.H_v, base4.H_k, base4.d, base4.decay, base4.update, base4.L)
    share = bench.extra_cfg("5tp8")
    base = CONFIGS[5]
    # one GPU's share under 8-way head sharding: every slot, a slice of the heads
    assert (share.num_slots, share.batch, share.H_v, share.H_k) == (base.num_slots, base.batch, 4, 2)
    assert (share.decay, share.update, share.state_dtype, share.L) == (base.decay, base.update, base.state_dtype,
                                                                       base.L)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["requested_gpus"] == 2 and "one GPU" in line["error"]
    assert "--gpus 1" in r.stderr


def _synthetic_rows():
    """Measured rows shaped as bench.summarize / time_window / time_flush give them."""
    from workloads import CONFIGS
    head = {"workload": "gdn_b1_h32_d128", "kernel": "deltalog", "batch": 1, "state": "f32", "value_tile": 16,
            "stream_ceiling": {"GBps": 1234.5678}, "frac_of_stream_ceiling": 0.55,
            "head_steps_per_s": 8.75e6, "tokens_per_s": 2.73e5, "ms_per_step": 3.66e-3, "decode_GBps": 680.1,
            "decode_frac_of_8TBps": 0.085, "decode_bytes_per_launch": 2.49e6, "decode_launch_us": 3.66,
            "decode_launch_source": "graph replay, back-to-back launches"}
    eager = dict(head, kernel="eager", ms_per_step=3.0e-3, head_steps_per_s=1.07e7, decode_GBps=1400.0)
    eager.pop("stream_ceiling")
    extras = []
    for tag in ("1", "3", "4", "5", "5tp8", "g64", "g128", "g256", "g512"):
        c = bench.extra_cfg(tag)
        for k, us in (("deltalog", 50.123456), ("eager", 90.987654)):
            extras.append({"workload": c.name, "kernel": k, "batch": c.batch, "state": c.state_dtype,
                           "value_tile": 128, "decode_launch_us": us, "decode_GBps": 5712.345678,
                           "decode_frac_of_8TBps": 0.714043, "head_steps_per_s": 1.234567e8, "rotated_pools": 4,
                           "long_field_that_stays_in_the_detail": "x" * 500,
                           "stream_ceiling": {"GBps": 6234.56789, "us": 40.1234, "blocks": 8192},
                           "frac_of_stream_ceiling": 0.9162345})
    windows = [{"workload": "gdn_b1_h32_d128", "W": w, "us_per_step": 0.71, "speedup_per_step_vs_decode": 5.1}
               for w in (16, 64, 256)]
    flushes = [{"workload": "gdn_b256_h32_d128", "launch_us": 205.9, "frac_of_8TBps": 0.71}]
    cpu = {"value": 4.0e4, "unit": "head-steps/s", "cores": 1, "kind": "oracle",
           "sample": "64 steps of gdn_b1_h32_d128 (all 32 slot-heads each), fp64 NumPy eager recurrence, 12.0 s wall",
           "cpu_model": "some CPU", "blas_threads": 1}
    return CONFIGS[2], head, eager, extras, windows, flushes, cpu


def test_stdout_line_is_compact_and_parses():
    cfg, head, eager, extras, windows, flushes, cpu = _synthetic_rows()
    steps = bench.cycle_steps(1, cfg.L, 20)
    line = bench.make_line(cfg, 1, steps, 5, 20, head, eager, extras, windows, flushes, cpu, 2629074.0,
                           "profiles/traffic_gdn_b1_h32_d128_rot1.json", "0123456789abcdef")
    text = json.dumps(line, separators=(",", ":"))
    assert len(text.encode()) <= 4096, len(text)
    back = json.loads(text)
    assert back["steps"] == 32 and back["steps_requested"] == 20 and back["warmup"] == 5
    assert back["dtype"] == "f32" and back["config"]["workload"] == cfg.name
    for k in ("metric", "value", "unit", "ms_per_step", "roofline", "cpu_baseline", "eager_baseline", "workloads"):
        assert k in back
    rf = back["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert set(back["cpu_baseline"]) == {"value", "unit", "cores", "kind", "sample"}
    names = [w["w"] for w in back["workloads"]]
    assert len(names) == 9 and len(set(names)) == 9
    assert all("x_eager" in w and "frac" in w and "of_ceil" in w for w in back["workloads"])


def test_decode_grid_matches_the_launch():
    from workloads import CONFIGS
    assert bench.decode_grid(CONFIGS[2], 16) == (256, 256)
    assert bench.decode_grid(CONFIGS[3], 64) == (2048, 128)
    assert bench.decode_grid(CONFIGS[5], 128) == (8192, 256)
    assert bench.decode_grid(CONFIGS[1], 16) == (2, 64)


def test_decode_kernel_names_the_launched_kernel():
    import dataclasses
    from workloads import CONFIGS
    # the launcher's rule (narrow tiles, scalar or no decay, key chunks and
    # value-side factor that fit the lane layout); the kernel traces name the
    # same kernels for workloads 1 and 2
    assert bench.decode_kernel(CONFIGS[2], 16) == "dl_small_kernel"
    assert bench.decode_kernel(CONFIGS[2], 32) == "dl_small_kernel"
    assert bench.decode_kernel(CONFIGS[2], 64) == "dl_step_kernel"
    assert bench.decode_kernel(CONFIGS[4], 16) == "dl_step_kernel"      # per-key decay
    assert bench.decode_kernel(CONFIGS[1], 16) == "dl_small_kernel"     # d = 16, fp32
    assert bench.decode_kernel(dataclasses.replace(CONFIGS[1], in_dtype="bf16"), 16) == "dl_step_kernel"
    assert bench.decode_kernel(CONFIGS[5], 128) == "dl_step_kernel"
    assert bench.decode_kernel(CONFIGS[5], 32) == "dl_small_kernel"     # bf16 tile, fp32 b: 8 x 4 bytes
    # d = 32, bf16 inputs, 32-column tile: plain LA keeps b in bf16 (16 x 2
    # bytes per lane), the delta rule in fp32 (16 x 4 bytes, over the limit)
    assert bench.decode_kernel(dataclasses.replace(CONFIGS[1], d=32, in_dtype="bf16"), 32) == "dl_small_kernel"
    assert bench.decode_kernel(dataclasses.replace(CONFIGS[2], d=32, in_dtype="bf16"), 32) == "dl_step_kernel"
    assert bench.decode_kernel(dataclasses.replace(CONFIGS[2], d=64), 32) == "dl_small_kernel"


def test_line_dtype_names_the_storage_of_16_bit_workloads():
    from workloads import CONFIGS
    assert bench.line_dtype(CONFIGS[2]) == "f32"
    assert bench.line_dtype(CONFIGS[5]).startswith("f32") and "bf16" in bench.line_dtype(CONFIGS[5])


def test_traffic_averages_the_most_dispatched_matching_kernel(tmp_path):
    # counter CSVs as rocprofv3 writes them: a torch conversion kernel whose
    # name also contains "_kernel<" ran 70 times, the decode kernel 200 times;
    # averaging the last 64 dispatches must not let the two tie
    from linear_attention_recurrent_dl_amd.rocprof_summary import traffic
    conv = "void at::native::vectorized_elementwise_kernel<4, bfloat16_copy_kernel_cuda>(int)"
    dec = "void dl::dl_step_kernel<128, 128, 2, true, float, unsigned short, 0>(int, int, int, unsigned int)"
    copy = "__amd_rocclr_copyBuffer"

    def write(path, counter, conv_v, dec_first, dec_last, copy_v):
        rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        did = 0
        for _ in range(70):
            did += 1
            rows.append(f'{did},"{conv}",{counter},{conv_v}')
        did += 1
        rows.append(f'{did},"{copy}",{counter},{copy_v}')
        for i in range(200):
            did += 1
            rows.append(f'{did},"{dec}",{counter},{dec_first if i < 136 else dec_last}')
        path.write_text("\n".join(rows) + "\n")

    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    write(fp, "FETCH_SIZE", 1.0, 999.0, 100.0, 512.0)     # copy of 1 KiB reads half: scale 2
    write(wp, "WRITE_SIZE", 1.0, 999.0, 10.0, 1024.0)
    t = traffic(str(fp), str(wp), "_kernel<", 1024 * 1024, last=64)
    assert t["kernel"] == dec and t["dispatches"] == 64
    assert t["hbm_fetch_bytes_per_launch"] == 100.0 * 1024 * 2
    assert t["hbm_write_bytes_per_launch"] == 10.0 * 1024


def test_trace_phases_sorts_dispatches_by_live_length(tmp_path):
    # two timed replays of 3 pools x L = 4 steps, pools decoded in turn; pool p
    # starts each replay at phase p (its merge is its (3 - p)-th dispatch),
    # and a dispatch starting from n entries lasts 10 + n (merge: 100) ns;
    # earlier dispatches of the kernel (warm-up) and other kernels are ignored
    from linear_attention_recurrent_dl_amd.rocprof_summary import trace_phases
    R, L = 3, 4
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0
    for _ in range(5):                             # warm-up dispatches of the same kernel
        rows.append(f'"k<1>",{t},{t + 7}')
        t += 1000
    for _ in range(2):
        for step in range(R * L):
            p, k = step % R, step // R
            n = (p + k) % L
            rows.append(f'"other",{t},{t + 5}')
            t += 1000
            rows.append(f'"k<1>",{t},{t + (100 if n == L - 1 else 10 + n)}')
            t += 1000
    path = tmp_path / "tr.csv"
    path.write_text("\n".join(rows) + "\n")
    by = trace_phases(str(path), "k<1>", R, L, 2)
    assert sorted(by) == [0, 1, 2, 3]
    assert all(len(v) == 2 * R for v in by.values())
    assert by[3] == [100] * (2 * R)
    for n in range(L - 1):
        assert by[n] == [10 + n] * (2 * R)
