"""Host logic of bench.py, on the CPU: the algorithmic byte count, the kernel the
library picks, and the profile summaries built from rocprofv3 CSV files (small
synthetic files here; the summaries are written to a temporary folder)."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GROUP = "_ZN12_GLOBAL__N_120rope_qk_group_kernelIDF16bLi8ELb0ELb0ELb0ELb0ELi1EEEvPT_S2_"
COPY = "__amd_rocclr_copyBuffer"


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for kernel, counter, value in rows:
            wr.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def _trace_csv(path, durations_ns, kernel=GROUP, grid=5242880):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X",
              "Workgroup_Size_X", "VGPR_Count", "LDS_Block_Size"]
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=fields)
        wr.writeheader()
        t = 1000
        for d in durations_ns:
            wr.writerow({"Kernel_Name": kernel, "Start_Timestamp": t, "End_Timestamp": t + d,
                         "Grid_Size_X": grid, "Workgroup_Size_X": 64, "VGPR_Count": 24,
                         "LDS_Block_Size": 2048})
            wr.writerow({"Kernel_Name": COPY, "Start_Timestamp": t, "End_Timestamp": t + 7,
                         "Grid_Size_X": 64, "Workgroup_Size_X": 64, "VGPR_Count": 8,
                         "LDS_Block_Size": 0})
            t += d + 100


def test_algorithmic_bytes():
    w = workloads.get("qwen3_4b_packed")
    assert bench.algorithmic_bytes_per_launch(w) == 2 * 16384 * (32 + 8) * 128 * 2 == 335544320
    p = workloads.get("qwen3_8b_padded")  # only the valid tokens count
    assert bench.algorithmic_bytes_per_launch(p) == 2 * p.valid_tokens * 40 * 128 * 2
    assert p.valid_tokens < p.T
    # the 524288-token pass is 8 launches: per-launch bytes are an eighth of the pass's
    w5 = workloads.get("long_ctx_512k")
    assert bench.algorithmic_bytes_per_pass(w5) == 2 * 524288 * 40 * 128 * 2
    assert bench.algorithmic_bytes_per_launch(w5) == bench.algorithmic_bytes_per_pass(w5) / 8


def _shape(T, Hq, Hkv, D=128, dtype="bf16"):
    return workloads.Workload(f"s{T}", 91, T, Hq, Hkv, D, dtype, 1e6, np.array([0, T], dtype=np.int32))


def test_launch_pieces():
    """The library's rule for issuing a long row-group pass as several launches:
    Q-heavy shapes (gq >= 4 gk) of 2 x 327680 workgroups or more, in launches of
    about 327680 workgroups over token ranges starting at multiples of 8."""
    assert bench.launch_pieces(workloads.get("long_ctx_512k")) == [65536] * 8   # 5 groups/token
    assert bench.launch_pieces(workloads.get("qwen3_4b_packed")) == [16384]
    assert bench.launch_pieces(workloads.get("qwen3_32b_packed")) == [32768]  # 294912 workgroups
    assert bench.launch_pieces(_shape(131072, 32, 8)) == [65536, 65536]        # exactly 2 x 327680
    assert bench.launch_pieces(_shape(131071, 32, 8)) == [131071]              # one workgroup short
    assert bench.launch_pieces(_shape(262144, 64, 8)) == [32768] * 8           # 9 groups/token
    assert bench.launch_pieces(_shape(524288, 16, 8)) == [524288]              # gq = 2 gk: never split
    assert bench.launch_pieces(_shape(524288, 32, 8), tokens_per_wave=1) == [524288]  # token kernel
    # ragged: 200003 tokens x 5 groups -> 4 launches of ceil(200003 / 4) rounded up to 8
    pieces = bench.launch_pieces(_shape(200003, 32, 8))
    assert pieces == [50008, 50008, 50008, 49979] and sum(pieces) == 200003
    assert all(p % 8 == 0 for p in pieces[:-1])
    # D = 64 in bf16: 16 rows per group, so 32 + 8 heads are 2 + 1 groups (gq < 4 gk)
    assert bench.launch_pieces(_shape(524288, 32, 8, D=64)) == [524288]
    # a compact padded launch counts rotated tokens
    pad = workloads.get("qwen3_8b_padded")
    assert bench.launch_pieces(pad) == [pad.valid_tokens]
    assert bench.launch_pieces(pad, "seqused") == [pad.T]


def test_kernel_choice():
    assert bench.rope_kernel_name(workloads.get("qwen3_4b_packed"), 0) == "rope_qk_group_kernel"
    assert bench.rope_kernel_name(workloads.get("qwen3_4b_packed"), 1) == "rope_qk_kernel"
    pad = workloads.get("qwen3_8b_padded")
    assert bench.rope_kernel_name(pad, 0) == "rope_qk_group_kernel"          # compact launch
    assert bench.rope_kernel_name(pad, 0, "seqused") == "rope_qk_kernel"
    assert bench.compact_launch(pad) and not bench.compact_launch(workloads.get("qwen3_4b_packed"))
    # grid of the compact launch: the rotated tokens' row groups only
    assert bench.expected_grid_threads(pad) == [pad.valid_tokens * 5 * 64]
    assert bench.expected_grid_threads(pad, "seqused") == [pad.T * 64]
    assert bench.expected_grid_threads(workloads.get("long_ctx_512k")) == [65536 * 5 * 64] * 8


def test_glu_pieces():
    """The library's rule for issuing a long GLU call as several launches: 65536
    workgroups (of 1024 16-byte chunks) or more, in launches of about 32768."""
    assert bench.glu_pieces(workloads.glu_get("glu_qwen3_4b")) == [19456]
    assert bench.glu_pieces(workloads.glu_get("glu_qwen3_8b")) == [12831]
    assert bench.glu_pieces(workloads.glu_get("glu_tiny")) == [1]
    assert bench.glu_pieces(workloads.glu_get("glu_long_512k")) == [32768] * 19


def test_staged_head_sizes():
    """Head sizes whose row halves are not whole 128-byte lines, or whose chunk count
    is not a power of two, take the row-group kernel's staged instance when the
    chunks are 16 bytes wide."""
    for D, dtype, nc, staged in ((128, "bf16", 8, False), (256, "bf16", 16, False),
                                 (512, "bf16", 32, False), (96, "bf16", 6, True),
                                 (80, "bf16", 5, True), (112, "f16", 7, True),
                                 (160, "bf16", 10, True), (64, "bf16", 4, True),
                                 (48, "bf16", 3, True), (64, "f32", 8, False)):
        w = _shape(1024, 32, 8, D=D, dtype=dtype)
        assert bench.chunks_per_half_row(w) == nc and bench.chunk_bytes(w) == 16
        assert bench.rope_kernel_name(w, 0) == "rope_qk_group_kernel"
        assert bench.staged_geometry(w) is staged, D
        steps = 2 if D == 512 else 1  # half rows of more than 128 elements: two row steps
        assert bench.group_steps(w) == steps
        assert bench.rope_kernel_instance(w, False).endswith(f"ELb{int(staged)}ELi{steps}E")
    # 11 to 15 chunks per half row: the staged instance with two steps
    for D, dtype, nc, rows in ((176, "bf16", 11, 8), (192, "bf16", 12, 10), (96, "f32", 12, 10),
                               (208, "f16", 13, 8), (224, "bf16", 14, 8), (240, "bf16", 15, 8)):
        w = _shape(1024, 32, 8, D=D, dtype=dtype)
        assert bench.chunks_per_half_row(w) == nc and bench.rope_kernel_name(w, 0) == "rope_qk_group_kernel"
        assert bench.staged_geometry(w) and bench.group_steps(w) == 2, D
        assert bench.rows_per_workgroup(w) == rows, D
        assert bench.rope_kernel_instance(w, False).endswith("ELb1ELi2E")
    # more chunks that do not divide 64 (too few rows even with two steps): the token kernel
    for D, dtype in ((272, "bf16"), (384, "bf16"), (176, "f32"), (320, "bf16")):
        w = _shape(1024, 32, 8, D=D, dtype=dtype)
        assert bench.rope_kernel_name(w, 0) == "rope_qk_kernel", D
    # D = 100 in bf16: 100-byte half rows, 4-byte chunks, nc = 25: the token kernel
    w = _shape(1024, 32, 8, D=100)
    assert bench.chunk_bytes(w) == 4 and bench.rope_kernel_name(w, 0) == "rope_qk_kernel"
    # D = 96 bf16, 32 + 8 heads: 10 rows per group, 4 + 1 groups per token
    w = _shape(131072, 32, 8, D=96)
    assert bench.expected_grid_threads(w) == [65536 * 5 * 64] * 2


def test_group_rows_whole_lines(tmp_path):
    """Rows per row group: 64 * steps // nc rounded down so that a group of 16-byte
    chunks spans whole 128-byte lines, when at least 5/8 of the lane slots stay busy.
    The library's group_rows (compiled from its source with g++), bench.py's mirror
    and a brute force over the definition agree for every nc and step count; D = 112 and 48 take aligned groups,
    D = 144 keeps 7 rows."""
    def brute(nc, steps=1):
        top = 64 * steps // nc
        whole = [r for r in range(top, 0, -1) if (r * nc * 32) % 128 == 0]
        return whole[0] if whole and 8 * whole[0] * nc >= 5 * 64 * steps else top
    src_text = open(os.path.join(ROOT, "packed_varlen_rotary_rope_amd", "csrc", "rope_qk.hip")).read()
    i = src_text.index("__host__ __device__ inline uint32_t group_rows(uint32_t nc, uint32_t steps = 1) {")
    j = src_text.index("\n}\n", i) + 3
    src = tmp_path / "group_rows.cpp"
    src.write_text("#include <cstdint>\n#include <cstdio>\n#define __host__\n#define __device__\n"
                   + src_text[i:j]
                   + "int main() { for (uint32_t nc = 1; nc <= 64; ++nc) printf(\"%u %u\\n\", "
                     "group_rows(nc), group_rows(nc, 2)); }\n")
    exe = tmp_path / "group_rows"
    subprocess.run(["g++", "-O2", "-std=c++17", "-o", str(exe), str(src)], check=True)
    lib = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    for nc in range(1, 65):
        assert lib[2 * (nc - 1)] == bench.group_rows(nc) == brute(nc), nc
        assert lib[2 * nc - 1] == bench.group_rows(nc, 2) == brute(nc, 2), nc
    # two steps: D = 192 (nc = 12) 10 rows, D = 144 (nc = 9) 12, D = 512 (nc = 32) 4
    assert [bench.group_rows(nc, 2) for nc in (9, 11, 12, 13, 15, 32)] == [12, 8, 10, 8, 8, 4]
    assert [bench.group_rows(nc) for nc in (3, 5, 6, 7, 9, 10)] == [20, 12, 10, 8, 7, 6]
    for nc in (1, 2, 4, 8, 16, 32, 64):
        assert bench.group_rows(nc) == 64 // nc
    # D = 112 bf16, 32 + 8 heads: 8 rows per group, 4 + 1 groups per token
    assert bench.expected_grid_threads(_shape(1000, 32, 8, D=112)) == [1000 * 5 * 64]
    # D = 48, 40 + 8 heads: 20 rows, 2 + 1 groups; D = 144, 14 + 2 heads: 7 rows, 2 + 1
    assert bench.expected_grid_threads(_shape(1000, 40, 8, D=48)) == [1000 * 3 * 64]
    assert bench.expected_grid_threads(_shape(1000, 14, 2, D=144)) == [1000 * 3 * 64]


def test_row_steps(tmp_path):
    """Two row steps per row-group workgroup for half rows of more than 128 elements
    in 16-byte chunks (D = 512) and for staged groups of 11 to 15 chunks per half row,
    one otherwise: the library's group_steps and staged_two_steps (compiled from its
    source with g++) and bench.py's mirror agree; the grid follows."""
    src_text = open(os.path.join(ROOT, "packed_varlen_rotary_rope_amd", "csrc", "rope_qk.hip")).read()
    parts = []
    for head in ("bool staged_two_steps(int32_t nc, int32_t chunk_bytes) {",
                 "int32_t group_steps(int32_t nc, int32_t half, int32_t chunk_bytes) {"):
        i = src_text.index(head)
        parts.append(src_text[i:src_text.index("\n}\n", i) + 3])
    src = tmp_path / "group_steps.cpp"
    src.write_text("#include <cstdint>\n#include <cstdio>\n" + "".join(parts)
                   + "int main() { for (int nc = 1; nc <= 64; ++nc) for (int h = 8; h <= 256; h *= 2)"
                   " for (int b = 2; b <= 16; b *= 2)"
                   " printf(\"%d %d %d %d\\n\", nc, h, b, group_steps(nc, h, b)); }\n")
    exe = tmp_path / "group_steps"
    subprocess.run(["g++", "-O2", "-std=c++17", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    for line in out.split("\n"):
        if not line:
            continue
        nc, half, cb, steps = (int(x) for x in line.split())
        assert steps == (2 if cb == 16 and (half > 128 or 11 <= nc <= 15) else 1), line
    for D, dtype, steps, rows in ((512, "bf16", 2, 4), (512, "f16", 2, 4), (512, "f32", 2, 2),
                                  (256, "bf16", 1, 4), (256, "f32", 1, 2), (128, "bf16", 1, 8),
                                  (192, "bf16", 2, 10), (176, "f16", 2, 8), (96, "f32", 2, 10)):
        w = _shape(1000, 7, 3, D=D, dtype=dtype)
        assert bench.group_steps(w) == steps and bench.rows_per_workgroup(w) == rows, D
        groups = -(-7 // rows) + -(-3 // rows)
        assert bench.expected_grid_threads(w) == [1000 * groups * 64], (D, dtype)
    assert bench.head_geometry(_shape(1000, 8, 8, D=512)) == "row-group, 2 rows x 2"
    assert bench.head_geometry(_shape(1000, 16, 16, D=192)) == "staged, 10 rows, 2 steps"


def test_kernel_instance_names():
    """The mangled-name fragments the summaries filter rocprofv3 records by."""
    w5, w2 = workloads.get("long_ctx_512k"), workloads.get("qwen3_4b_packed")
    assert bench.needs_long_index(w5) and not bench.needs_long_index(w2)
    assert bench.rope_kernel_instance(w5, True) == "rope_qk_group_kernelIDF16bLi8ELb1ELb0ELb0ELb0ELi1E"
    assert bench.rope_kernel_instance(w2, False) in GROUP
    assert bench.rope_kernel_instance(workloads.get("tiny_packed"), False) == \
        "rope_qk_group_kernelIfLi4ELb0ELb0ELb0ELb1ELi1E"  # D = 16 in fp32: staged
    pad = workloads.get("qwen3_8b_padded")
    assert bench.rope_kernel_instance(pad, False) == "rope_qk_group_kernelIDF16bLi8ELb0ELb0ELb1ELb0ELi1E"
    assert bench.rope_kernel_instance(pad, False, "seqused") == \
        "rope_qk_kernelIDF16bLi8ELb0ELb0E"
    assert bench.rope_instance_names(pad, False)[1] == \
        "rope_qk_group_kernel<__bf16, 8, false, false, true, false, 1>"
    assert bench.rope_instance_names(w5, True)[1] == \
        "rope_qk_group_kernel<__bf16, 8, true, false, false, false, 1>"


def test_linear_fit():
    T = np.array([1000, 2000, 8000, 64000])
    t0, b = bench.linear_fit(T, 1.5 + 0.003 * T)
    assert abs(t0 - 1.5) < 1e-9 and abs(b - 0.003) < 1e-12


def test_traffic_summary_and_hash_check(tmp_path, monkeypatch):
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(out))
    kib = 1024.0
    # the copy reads 1 GiB and writes 1 GiB; its counters read half and all of that
    _counter_csv(str(tmp_path / "cf.csv"), [(COPY, "FETCH_SIZE", 2 ** 30 / kib / 2)])
    _counter_csv(str(tmp_path / "cw.csv"), [(COPY, "WRITE_SIZE", 2 ** 30 / kib)])
    half = 335544320 / 2 / kib
    _counter_csv(str(tmp_path / "f.csv"), [(GROUP, "FETCH_SIZE", half / 2)] * 3)
    _counter_csv(str(tmp_path / "w.csv"), [(GROUP, "WRITE_SIZE", half)] * 3)
    bench.write_traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), "cmd")
    text = out.read_text()
    assert "fetch_scale: 2.00000" in text and "write_scale: 1.00000" in text
    assert "traffic_over_algorithmic: 1.0000" in text
    assert bench.read_traffic(str(out)) == 335544320
    # a summary taken on other kernel sources is not used
    out.write_text(text.replace(bench.kernel_source_hash(bench.ROPE_SOURCES), "0" * 16))
    assert bench.read_traffic(str(out)) is None


def test_traffic_summary_request_counts(tmp_path, monkeypatch):
    """The second counter family: bytes from request counts x request sizes by the
    counters' definitions (no calibration), for the long-context (64-bit) instance."""
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(out))
    w = workloads.get("long_ctx_512k")
    bpl = bench.algorithmic_bytes_per_launch(w)
    long_k = "_ZN12_GLOBAL__N_120rope_qk_group_kernelIDF16bLi8ELb1ELb0ELb0ELb0ELi1EEEvPT_S2_"
    kib = 1024.0
    for name, ctr, val in (("cf", "FETCH_SIZE", 2 ** 30 / kib / 2), ("cw", "WRITE_SIZE", 2 ** 30 / kib)):
        _counter_csv(str(tmp_path / f"{name}.csv"), [(COPY, ctr, val)])
    _counter_csv(str(tmp_path / "f.csv"), [(long_k, "FETCH_SIZE", bpl / 2 / kib / 2)])
    _counter_csv(str(tmp_path / "w.csv"), [(long_k, "WRITE_SIZE", bpl / 2 / kib)])
    # all reads are 128-byte requests, all writes 64-byte ones
    def rd(n):
        return [("TCC_EA0_RDREQ_sum", n), ("TCC_EA0_RDREQ_32B_sum", 0),
                ("TCC_EA0_RDREQ_128B_sum", n), ("TCC_BUBBLE_sum", 0)]
    def wr(n):
        return [("TCC_EA0_WRREQ_sum", n), ("TCC_EA0_WRREQ_64B_sum", n)]
    _counter_csv(str(tmp_path / "er.csv"), [(long_k, c, v) for c, v in rd(bpl / 2 / 128)]
                 + [(GROUP, c, 1.0) for c, v in rd(1)])
    _counter_csv(str(tmp_path / "ew.csv"), [(long_k, c, v) for c, v in wr(bpl / 2 / 64)])
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>"
    _counter_csv(str(tmp_path / "cer.csv"), [(fill, c, v) for c, v in rd(300)]
                 + [(COPY, c, v) for c, v in rd(2 ** 30 / 128)])
    _counter_csv(str(tmp_path / "cew.csv"), [(COPY, c, v) for c, v in wr(2 ** 30 / 64)])
    bench.write_traffic_summary(*(str(tmp_path / f"{n}.csv") for n in ("f", "w", "cf", "cw")),
                                "cmd", workload="long_ctx_512k",
                                ea=[str(tmp_path / f"{n}.csv") for n in ("er", "ew", "cer", "cew")])
    text = out.read_text()
    assert "rope_qk_group_kernelIDF16bLi8ELb1ELb0E" in text
    assert "traffic_over_algorithmic: 1.0000" in text
    assert "ea_traffic_over_algorithmic: 1.0000" in text
    assert "ea_copy_read_bytes_for_1GiB: 1073741824 (x1.0000)" in text
    assert bench.read_traffic(str(out)) == bpl


def test_sweep_summary(tmp_path, monkeypatch):
    out = tmp_path / "sweep.txt"
    monkeypatch.setattr(bench, "SWEEP_FILE", str(out))
    sizes = [2048, 16384, 65536]
    pieces = {2048: 1, 16384: 1, 65536: 2}  # the largest size as two launches per pass
    rows, trace = [], []
    for T in sizes:
        us = 1.5 + 0.003 * T
        rows.append({"T": T, "avg_pass_us": us + 0.1, "launches_per_pass": pieces[T],
                     "torch_inplace_us": 2 + 0.0035 * T, "GBps": 0.0, "index": "32-bit"})
        trace.append((T, int(us * 1e3)))
    js = {"bytes_per_token": 20480, "rows": rows}
    for key in ("avg_pass_us", "torch_inplace_us"):
        t0, b = bench.linear_fit(sizes, [r[key] for r in rows])
        js[f"fit_{key}"] = {"t0_us": t0, "us_per_token": b,
                            "asymptotic_GBps": 20480 / (b * 1e-6) / 1e9}
    (tmp_path / "sweep.json").write_text("noise\n" + bench.json.dumps(js) + "\n")
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]
    os.makedirs(tmp_path / "tr")
    with open(tmp_path / "tr" / "x_kernel_trace.csv", "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=fields)
        wr.writeheader()
        clock = 0
        # each size: one run of RoPE dispatches (3 passes) between torch's own kernels
        for T, ns in trace:
            n = pieces[T]
            for _ in range(3 * n):
                wr.writerow({"Kernel_Name": GROUP, "Start_Timestamp": clock,
                             "End_Timestamp": clock + ns // n, "Grid_Size_X": T // n * 5 * 64})
                clock += ns
            wr.writerow({"Kernel_Name": COPY, "Start_Timestamp": clock, "End_Timestamp": clock + 5,
                         "Grid_Size_X": 64})
            clock += 10
    bench.write_sweep_summary(str(tmp_path), "cmd")
    text = out.read_text()
    assert "fit, RoPE kernel, trace averages, all sizes: t = 1.50 us + T x 3.0000 ns" in text, text
    assert "fit, RoPE kernel, trace averages, T <= 65536: t = 1.50 us + T x 3.0000 ns" in text


def test_head_shapes_summary(tmp_path, monkeypatch):
    """The head-shape survey's summary: one row per shape with its geometry (the
    library's kernel choice and rows per group, as bench.py mirrors it), pass time,
    GB/s and the torch reference, from a synthetic JSON line."""
    import json
    out = tmp_path / "shapes.txt"
    monkeypatch.setattr(bench, "HEAD_SHAPES_FILE", str(out))
    rows = []
    for Hq, Hkv, D, dtype in bench.HEAD_SHAPES:
        w = bench.head_shape_workload(Hq, Hkv, D, dtype)
        us = bench.algorithmic_bytes_per_pass(w) / 6.4e9 * 1e3  # 6.4 TB/s
        rows.append({"Hq": Hq, "Hkv": Hkv, "D": D, "dtype": dtype, "T": w.T,
                     "geometry": bench.head_geometry(w), "launches_per_pass": 1,
                     "avg_pass_us": us, "GBps": 6400.0, "frac": 0.8,
                     "torch_inplace_us": 1.2 * us, "frac_of_ceiling": 1.2})
    js = tmp_path / "shapes.json"
    js.write_text("noise\n" + json.dumps({"head_shapes": "synthetic", "rows": rows}) + "\n")
    bench.write_head_shapes_summary(str(js), "python R/bench.py --head-shapes")
    text = out.read_text()
    body = [ln for ln in text.splitlines() if ln and not ln.startswith("#")]
    assert len(body) == 1 + len(bench.HEAD_SHAPES)
    assert "python R/bench.py --head-shapes" in text
    assert f"kernel_source_sha256_16: {bench.kernel_source_hash()}" in text
    assert any("staged, 8 rows" in ln and " 112 " in ln for ln in body)      # D = 112
    assert any("staged, 10 rows, 2 steps" in ln and " 192 " in ln for ln in body)  # D = 192
    assert all("80.0%" in ln for ln in body[1:])


def test_trace_summary(tmp_path, monkeypatch):
    out = tmp_path / "trace.txt"
    monkeypatch.setattr(bench, "trace_summary_path", lambda workload: str(out))
    durations = [50000, 52000, 54000, 60000]
    _trace_csv(str(tmp_path / "t.csv"), durations)
    bench.write_trace_summary(str(tmp_path / "t.csv"), "qwen3_4b_packed", "cmd")
    text = out.read_text()
    assert "dispatches: 4" in text
    mean = float(np.mean(durations)) / 1e3
    gbps = 335544320 / (mean * 1e-6) / 1e9
    assert f"average: {mean:.2f} us -> {gbps:.0f} GB/s" in text
    assert "minimum: 50.00 us" in text and "maximum: 60.00 us" in text
    assert "static LDS only" in text
    assert "launches_per_pass" not in text


def test_trace_summary_multi_launch_pass(tmp_path, monkeypatch):
    """The 524288-token pass is 8 launches of 65536 tokens: per-launch bytes are an
    eighth of the pass's, and tokens/s count whole passes."""
    out = tmp_path / "trace.txt"
    monkeypatch.setattr(bench, "trace_summary_path", lambda workload: str(out))
    long_k = "_ZN12_GLOBAL__N_120rope_qk_group_kernelIDF16bLi8ELb1ELb0ELb0ELb0ELi1EEEvPT_S2_"
    durations = [200000] * 16
    _trace_csv(str(tmp_path / "t.csv"), durations, kernel=long_k, grid=65536 * 5 * 64)
    bench.write_trace_summary(str(tmp_path / "t.csv"), "long_ctx_512k", "cmd")
    text = out.read_text()
    assert "launches_per_pass: 8 (tokens per launch: 65536)" in text
    assert "algorithmic_bytes_per_launch: 1342177280" in text
    gbps = 1342177280 / 200e-6 / 1e9
    assert f"average: 200.00 us -> {gbps:.0f} GB/s" in text
    assert f"valid_tokens_per_s_at_average: {524288 / (8 * 200e-6):.4g} per pass" in text
    # dispatches with another grid (another workload's launches) are not counted
    _trace_csv(str(tmp_path / "u.csv"), durations, kernel=long_k, grid=524288 * 5 * 64)
    with pytest.raises(SystemExit):
        bench.write_trace_summary(str(tmp_path / "u.csv"), "long_ctx_512k", "cmd")


def test_counters_summary(tmp_path, monkeypatch):
    out = tmp_path / "counters.txt"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(out))
    kib = 1024.0
    _counter_csv(str(tmp_path / "cf.csv"), [(COPY, "FETCH_SIZE", 2 ** 30 / kib / 2)])
    _counter_csv(str(tmp_path / "cw.csv"), [(COPY, "WRITE_SIZE", 2 ** 30 / kib)])
    base = {"SQ_WAVES": 1000, "SQ_INSTS_VALU": 200000, "SQ_INSTS_VALU_FMA_F64": 19000,
            "SQ_INSTS_SALU": 1, "SQ_INSTS_SMEM": 1, "SQ_INSTS_LDS": 5000, "SQ_INSTS_VMEM_RD": 6000,
            "SQ_INSTS_VMEM_WR": 2000, "SQ_LDS_BANK_CONFLICT": 0, "SQ_ACTIVE_INST_VALU": 256000,
            "GRBM_GUI_ACTIVE": 8000, "SQ_WAVE_CYCLES": 1000, "SQ_WAIT_INST_ANY": 1,
            "FETCH_SIZE": 100, "WRITE_SIZE": 100}
    for mode, valu in (("fly", 256000), ("table", 128000)):
        vals = dict(base, SQ_ACTIVE_INST_VALU=valu)
        _counter_csv(str(tmp_path / mode / "pmc1" / "bench_counter_collection.csv"),
                     [(GROUP, k, v) for k, v in vals.items()] * 2)
        _trace_csv(str(tmp_path / mode / "trace" / "bench_kernel_trace.csv"), [50000])
    bench.write_counters_summary(str(tmp_path / "fly"), str(tmp_path / "table"),
                                 str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), "cmd")
    line = [ln for ln in out.read_text().splitlines() if ln.startswith("VALU busy")][0]
    # 4 cycles x 256000 instructions over 1024 SIMDs x (8000 / 8) cycles = 100%
    assert line.split()[-3:] == ["100.0", "50.0", "x0.500"]
    fetch = [ln for ln in out.read_text().splitlines() if ln.startswith("HBM read")][0]
    assert "2.048e+05" in fetch  # 100 KiB x scale 2


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_source_hash_ignores_documentation(tmp_path, monkeypatch):
    """The profile hash follows the code and the build script, not their comments or
    docstrings: a comment edit keeps it, a code or flag edit changes it."""
    import shutil
    for name in bench.ROPE_SOURCES:
        dst = tmp_path / "pkg" / "csrc" / name
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.KERNEL_SRC, name), dst)
    monkeypatch.setattr(bench, "KERNEL_SRC", str(tmp_path / "pkg" / "csrc"))
    base = bench.kernel_source_hash()
    hip = tmp_path / "pkg" / "csrc" / "rope_qk.hip"
    text = hip.read_text()
    hip.write_text(text.replace("// ", "//  ", 5) + "\n/* a note */\n// another\n")
    assert bench.kernel_source_hash() == base
    hip.write_text(text.replace("constexpr int kBlock = 256;", "constexpr int kBlock = 128;"))
    assert bench.kernel_source_hash() != base
    hip.write_text(text)
    build = tmp_path / "pkg" / "build.py"
    code = build.read_text()
    build.write_text(code.replace('"""', '"""Edited docstring. ', 1) + "\n# a comment\n")
    assert bench.kernel_source_hash() == base
    build.write_text(code.replace("-amdgpu-kernarg-preload-count=13", "-amdgpu-kernarg-preload-count=8"))
    assert bench.kernel_source_hash() != base
