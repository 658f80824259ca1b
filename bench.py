"""Benchmark: fused packed-varlen QK-RoPE, forward + backward, on one MI355X.

One step = forward RoPE on (Q, K) plus backward RoPE on (dQ, dK) of one packed
batch: two launches of the fused kernel, every row of the hot path. Default
workload: the largest one, a single 524288-token sequence (Hq = 32, Hkv = 8,
D = 128, bf16, theta = 1e6; Q alone holds 2^31 elements, so the 64-bit offset
instance runs), standing in for the Unsloth page's 500K-token contexts. The same
JSON line carries per-workload results for the other workloads (region-timed
launches of the default path, with a torch in-place elementwise reference over
the same bytes), so one run covers every configuration.

Inputs are synthetic, seeded and resident in HBM before timing starts. Several
buffer sets are rotated so that the working set between two touches of the
same buffer exceeds the 256 MB Infinity Cache: every launch reads and writes
HBM, as a training step would.

Prints ONE JSON line (rank 0). `value` is tokens/s of whole steps (wall clock
around K steps, bracketed by synchronize). `roofline` uses the kernel's average
launch duration: the GPU time of the timed region, from one pair of HIP events
(timing-only, no system fence) recorded on the launch stream around it, divided
by its 2K launches (gaps between launches included). Per-launch minimum and
median come from events around single launches in a sampling pass after the
timed region. `traffic` comes from the committed rocprofv3 PMC
summary when it was taken on the current kernel source, else null.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload
(for the 524288-token sequence: the gathered rows of evenly spaced tokens).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

METRIC = "fused QK-RoPE fwd+bwd tokens/s and achieved HBM GB/s (% of peak), packed bf16"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
INFINITY_CACHE_BYTES = 256 * 2 ** 20
KERNEL_SRC = os.path.join(ROOT, "packed_varlen_rotary_rope_amd", "csrc")
HEADLINE_WORKLOAD = "long_ctx_512k"
# workloads timed beside the headline in the default run (every bf16 and fp32 one)
SUB_WORKLOADS = ["tiny_packed", "qwen3_4b_packed", "qwen3_8b_packed", "qwen3_8b_padded",
                 "qwen3_32b_packed", "long_ctx_512k"]


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"rope_qk_{workload}_traffic.txt")


TRAFFIC_FILE = traffic_path("qwen3_4b_packed")


# The sources each kernel is compiled from: a traffic summary taken on other
# sources does not describe the kernel being timed.
# what a kernel's code depends on: its sources and the build script (its flags)
ROPE_SOURCES = ["rope_qk.hip", "storage.h", "cr_sincos.h", "trig_constants.h", "fast_div.h",
                "../../include/rope_qk.h", "../build.py"]
GLU_SOURCES = ["glu.hip", "storage.h", "glu_constants.h", "../../include/glu.h",
               "../../include/rope_qk.h", "../build.py"]
GLU_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "glu_swiglu_qwen3_4b_traffic.txt")
# bf16, 16-byte chunks, SwiGLU, dense, 32-bit offsets: forward and backward instances
GLU_KERNEL_KEYS = {"fwd": "glu_kernelIDF16bLi8ELi0ELb0ELb1Ej", "bwd": "glu_kernelIDF16bLi8ELi0ELb1ELb1Ej"}


def glu_instance(code: int, bwd: int) -> str:
    """Mangled-name fragment of the bf16, 16-byte, dense GLU instance the library runs
    by default for this kind and pass (the tanh-GeGLU backward takes 64-bit offsets)."""
    index = "l" if (code == 2 and bwd) else "j"
    return f"glu_kernelIDF16bLi8ELi{code}ELb{bwd}ELb1E{index}"


def _code_text(name: str, raw: bytes) -> bytes:
    """The code of a source file without its comments, blank lines and (Python)
    docstrings, so that editing documentation does not invalidate a profile taken on
    the same code, while any change to code or build flags does."""
    text = raw.decode()
    if name.endswith(".py"):
        import ast
        tree = ast.parse(text)
        for node in ast.walk(tree):
            body = getattr(node, "body", None)
            if (isinstance(node, (ast.Module, ast.FunctionDef, ast.ClassDef)) and body and
                    isinstance(body[0], ast.Expr) and isinstance(body[0].value, ast.Constant) and
                    isinstance(body[0].value.value, str)):
                node.body = body[1:] or [ast.Pass()]
        return ast.dump(tree).encode()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln.strip()).encode()


def kernel_source_hash(sources=ROPE_SOURCES) -> str:
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(KERNEL_SRC, name), "rb") as fh:
            h.update(name.encode() + b"\0" + _code_text(name, fh.read()))
    return h.hexdigest()[:16]


def compact_launch(w: workloads.Workload, padded: str = "compact") -> bool:
    """Whether a padded workload (seqused) is launched compact: rope_qk_apply_padded
    with cu_valid and the host count of rotated tokens, the grid covering only them."""
    return w.seqused is not None and padded == "compact"


def rope_kernel_name(w: workloads.Workload, tokens_per_wave: int, padded: str = "compact") -> str:
    """The kernel the library picks for this call: row groups by default and for
    compact padded launches, one wave per token when the caller sets tokens per wave
    or passes seqused to the plain entry points."""
    if tokens_per_wave == 0 and group_geometry(w) and (w.seqused is None or
                                                       compact_launch(w, padded)):
        return "rope_qk_group_kernel"
    return "rope_qk_kernel"


def chunk_bytes(w: workloads.Workload) -> int:
    """The widest access (<= 16 bytes) that divides a half row, for contiguous
    aligned tensors (the library also checks strides and addresses)."""
    half_bytes = (w.D // 2) * w.elem_bytes
    b = 16
    while b > w.elem_bytes and half_bytes % b:
        b //= 2
    return b


def chunks_per_half_row(w: workloads.Workload) -> int:
    """nc: chunks per half row."""
    return (w.D // 2) * w.elem_bytes // chunk_bytes(w)


def group_geometry(w: workloads.Workload) -> bool:
    """Whether the row-group kernel takes this head size: nc divides 64, or the
    staged instance applies."""
    return 64 % chunks_per_half_row(w) == 0 or staged_geometry(w)


def staged_geometry(w: workloads.Workload) -> bool:
    """The row-group kernel's STAGED instance: 16-byte chunks, at most 10 per half row
    and not 8, or 11 to 15 with two steps (the library's staged_geometry)."""
    nc = chunks_per_half_row(w)
    return chunk_bytes(w) == 16 and ((nc <= 10 and nc != 8) or 11 <= nc <= 15)


def group_rows(nc: int, steps: int = 1) -> int:
    """Head rows per row group (the library's group_rows): 64 * steps // nc, rounded
    down to whole 128-byte lines of 16-byte chunks (rows * nc a multiple of 4) when
    that keeps at least 5/8 of the 64 * steps lane slots busy."""
    r = 64 * steps // nc
    a = r & ~3 if nc & 1 else r & ~1 if (nc & 3) == 2 else r
    return a if 8 * a * nc >= 5 * 64 * steps else r


def group_steps(w: workloads.Workload) -> int:
    """Row steps per row-group workgroup (the library's group_steps): 2 for half rows
    of more than 128 elements in 16-byte chunks (D = 512) and for staged groups of
    11 to 15 chunks per half row, else 1."""
    nc = chunks_per_half_row(w)
    two = chunk_bytes(w) == 16 and (w.D // 2 > 128 or 11 <= nc <= 15)
    return 2 if two else 1


def rows_per_workgroup(w: workloads.Workload) -> int:
    """Head rows one row-group workgroup rotates: group_rows(nc, group_steps)."""
    return group_rows(chunks_per_half_row(w), group_steps(w))


# The library's kPieceBlocks: a long pass of the row-group kernel on a Q-heavy shape
# is issued as consecutive launches of about this many workgroups.
PIECE_BLOCKS = 327680


def group_pieces(rows: int, w: workloads.Workload) -> list:
    """Tokens of each launch the row-group kernel is issued as over `rows` tokens of
    w's head shape: one launch, except that a pass of 2 x PIECE_BLOCKS workgroups or
    more, when Q holds at least 4x K's row groups, is issued as launches of about
    PIECE_BLOCKS workgroups over consecutive token ranges that start at multiples of
    8 tokens (the library's group_piece_tokens)."""
    rows_per_group = rows_per_workgroup(w)
    gq, gk = -(-w.Hq // rows_per_group), -(-w.Hkv // rows_per_group)
    blocks = rows * (gq + gk)
    if gq < 4 * gk or blocks < 2 * PIECE_BLOCKS:
        return [rows]
    n = -(-blocks // PIECE_BLOCKS)
    piece = (-(-rows // n) + 7) // 8 * 8
    return [min(piece, rows - t0) for t0 in range(0, rows, piece)]


def launch_pieces(w: workloads.Workload, padded: str = "compact", tokens_per_wave: int = 0) -> list:
    """Tokens (rotated tokens, for a compact launch) of each launch of one default
    pass, in order."""
    if rope_kernel_name(w, tokens_per_wave, padded) != "rope_qk_group_kernel":
        return [w.T]
    return group_pieces(w.valid_tokens if compact_launch(w, padded) else w.T, w)


def algorithmic_bytes_per_pass(w: workloads.Workload) -> int:
    """One read and one write of every rotated element of Q and K (or dQ and dK)."""
    return 2 * w.valid_tokens * (w.Hq + w.Hkv) * w.D * w.elem_bytes


def algorithmic_bytes_per_launch(w: workloads.Workload, padded: str = "compact") -> float:
    """The pass's bytes over its launches (an average where the last launch of a
    multi-launch pass is shorter)."""
    total, n = algorithmic_bytes_per_pass(w), len(launch_pieces(w, padded))
    return total // n if total % n == 0 else total / n


def read_traffic(path: str = TRAFFIC_FILE, sources=ROPE_SOURCES, field="hbm_bytes_per_launch"):
    """HBM bytes per launch from a committed PMC summary, if it matches the sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_0-9]+)\s*[:=]\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return int(float(kv[field]))
    except (KeyError, ValueError):
        return None


class HipEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it
    takes a timestamp on the stream without the system-scope cache writeback and
    invalidate of a default event, so the interval around one launch is close to
    the launch itself. Bound to the HIP runtime already mapped in this process
    (the one torch and the library use)."""

    _lib = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def lib(cls):
        if cls._lib is None:
            import ctypes
            paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps")
                            if "libamdhip64" in ln and ln.split()[-1].startswith("/")})
            if not paths:
                raise RuntimeError("no HIP runtime mapped in this process")
            lib = ctypes.CDLL(paths[0])
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._lib = lib
        return cls._lib

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        if self.lib().hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE):
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream: int):
        if self.lib().hipEventRecord(self._ev, stream):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        if self.lib().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._lib is not None and self._ev:
            self._lib.hipEventDestroy(self._ev)


def _dispatch_means(csv_path: str) -> dict:
    """Mean Counter_Value (KiB) per kernel name over the dispatches of a rocprofv3
    --pmc CSV."""
    import csv
    acc = {}
    with open(csv_path) as fh:
        for row in csv.DictReader(fh):
            acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _pmc_scaled(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, key):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the kernel whose name contains
    key, and the same counters for a plain 1 GiB device copy (written and read
    once), which give the scale from counter units to bytes."""
    copy_bytes = 2 ** 30

    def kernel(means):
        hits = [(k, v) for k, v in means.items() if key in k]
        if not hits:
            raise SystemExit(f"no dispatch of {key} in the counter file")
        return max(hits, key=lambda kv: kv[1][1])[1]

    def copy_kernel(means):
        return max(means.items(), key=lambda kv: kv[1][0])[1]  # the 1 GiB copy dominates

    f_k, nf = kernel(_dispatch_means(fetch_csv))
    w_k, nw = kernel(_dispatch_means(write_csv))
    f_c, _ = copy_kernel(_dispatch_means(copy_fetch_csv))
    w_c, _ = copy_kernel(_dispatch_means(copy_write_csv))
    f_scale = copy_bytes / (f_c * 1024.0)
    w_scale = copy_bytes / (w_c * 1024.0)
    return {"f_k": f_k, "w_k": w_k, "nf": nf, "nw": nw, "f_c": f_c, "w_c": w_c,
            "f_scale": f_scale, "w_scale": w_scale, "read": f_k * 1024.0 * f_scale,
            "write": w_k * 1024.0 * w_scale}


def _pmc_lines(m, bpl, prefix=""):
    return [
        f"{prefix}fetch_kib_per_dispatch: {m['f_k']:.1f}",
        f"{prefix}write_kib_per_dispatch: {m['w_k']:.1f}",
        f"{prefix}dispatches_counted: {m['nf']} {m['nw']}",
        f"{prefix}hbm_read_bytes_per_launch: {m['read']:.0f}",
        f"{prefix}hbm_write_bytes_per_launch: {m['write']:.0f}",
        f"{prefix}hbm_bytes_per_launch: {m['read'] + m['write']:.0f}",
        f"{prefix}algorithmic_bytes_per_launch: {bpl}",
        f"{prefix}traffic_over_algorithmic: {(m['read'] + m['write']) / bpl:.4f}",
    ]


def _write_summary(path, header, lines):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        fh.write("\n".join(header + lines) + "\n")
    print("\n".join(header + lines))


def _counter_means(csv_path: str) -> dict:
    """{kernel name: {counter: mean per dispatch}} over a rocprofv3 --pmc CSV that may
    hold several counters per dispatch."""
    acc = {}
    with open(csv_path) as fh:
        for row in csv.DictReader(fh):
            acc.setdefault(row["Kernel_Name"], {}).setdefault(row["Counter_Name"], []).append(
                float(row["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}


def _pick(means: dict, key: str | None) -> dict:
    """The counters of the kernel whose name contains key; key None means the 1 GiB
    device copy of --copy-calibration (the runtime's copy kernel, else the kernel with
    the largest readings: the fill that makes its source reads nothing)."""
    if key is None:
        copies = [d for k, d in means.items() if "copyBuffer" in k]
        if copies:
            return copies[0]
        return max(means.values(), key=lambda d: sum(d.values()))
    hits = [d for k, d in means.items() if key in k]
    if not hits:
        raise SystemExit(f"no dispatch of {key} in the counter file")
    return hits[0]


def ea_bytes(read: dict, write: dict) -> tuple:
    """HBM read and write bytes from the TCC-to-memory request counts, by the
    counters' definitions: a read request is 32, 64 or 128 bytes (TCC_EA0_RDREQ counts
    all, _32B and _128B the two sizes named), a write request 32 or 64 bytes
    (TCC_EA0_WRREQ all, _64B the large ones). No calibration enters."""
    rd, r32, r128 = (read[c] for c in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum",
                                       "TCC_EA0_RDREQ_128B_sum"))
    wr, w64 = write["TCC_EA0_WRREQ_sum"], write["TCC_EA0_WRREQ_64B_sum"]
    return 128 * r128 + 32 * r32 + 64 * (rd - r128 - r32), 64 * w64 + 32 * (wr - w64)


def write_traffic_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, command: str,
                          workload: str = "qwen3_4b_packed", ea=None):
    """HBM bytes per launch of the workload's default RoPE kernel instance from two PMC
    passes (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter reads
    for a plain 1 GiB device copy, as a small text summary that main() reads back.
    With ea = (read CSV, write CSV, copy read CSV, copy write CSV) of two more passes
    (TCC_EA0_RDREQ/_32B/_128B and TCC_BUBBLE; TCC_EA0_WRREQ/_64B), the bytes are also
    derived from the request counts by the counters' definitions, uncalibrated."""
    w = workloads.get(workload)
    key = rope_kernel_instance(w, needs_long_index(w))
    m = _pmc_scaled(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, key)
    bpl = algorithmic_bytes_per_launch(w)
    seq = "padded rows skipped via seqused" if w.seqused is not None else "packed"
    header = [
        f"# HBM traffic of the RoPE kernel instance {key}",
        f"# on the {w.name} workload (T={w.T}, {w.valid_tokens} valid tokens, {seq}; Hq={w.Hq},",
        f"# Hkv={w.Hkv}, D={w.D}, {w.dtype}), one launch = forward or backward over Q and K"
        + ("." if len(launch_pieces(w)) == 1 else
           f"\n# of one of the {len(launch_pieces(w))} token ranges a pass is issued as."),
        "# Two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) over the same bench",
        "# command, each counter scaled by its reading for a plain 1 GiB device copy.",
        f"# commands: {command}",
        f"copy_fetch_kib_for_1GiB: {m['f_c']:.1f}",
        f"copy_write_kib_for_1GiB: {m['w_c']:.1f}",
        f"fetch_scale: {m['f_scale']:.5f}",
        f"write_scale: {m['w_scale']:.5f}",
    ]
    lines = _pmc_lines(m, bpl)
    if ea is not None:
        kr, kw = _pick(_counter_means(ea[0]), key), _pick(_counter_means(ea[1]), key)
        cr, cw = _pick(_counter_means(ea[2]), None), _pick(_counter_means(ea[3]), None)
        k_read, k_write = ea_bytes(kr, kw)
        c_read, c_write = ea_bytes(cr, cw)
        lines += [
            "# second counter family: TCC-to-memory request counts x request size (uncalibrated)",
            f"ea_copy_read_bytes_for_1GiB: {c_read:.0f} (x{c_read / 2 ** 30:.4f})",
            f"ea_copy_write_bytes_for_1GiB: {c_write:.0f} (x{c_write / 2 ** 30:.4f})",
            f"ea_read_requests_per_launch: {kr['TCC_EA0_RDREQ_sum']:.0f} "
            f"(32B {kr['TCC_EA0_RDREQ_32B_sum']:.0f}, 128B {kr['TCC_EA0_RDREQ_128B_sum']:.0f}, "
            f"TCC_BUBBLE {kr.get('TCC_BUBBLE_sum', float('nan')):.0f})",
            f"ea_write_requests_per_launch: {kw['TCC_EA0_WRREQ_sum']:.0f} "
            f"(64B {kw['TCC_EA0_WRREQ_64B_sum']:.0f})",
            f"ea_hbm_read_bytes_per_launch: {k_read:.0f}",
            f"ea_hbm_write_bytes_per_launch: {k_write:.0f}",
            f"ea_traffic_over_algorithmic: {(k_read + k_write) / bpl:.4f}",
        ]
    lines.append(f"kernel_source_sha256_16: {kernel_source_hash(ROPE_SOURCES)}")
    _write_summary(traffic_path(w.name), header, lines)


def write_glu_traffic_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, command: str):
    """The same for the SwiGLU forward and backward kernels on glu_qwen3_4b."""
    w = workloads.glu_get("glu_qwen3_4b")
    header = [
        "# HBM traffic of glu_kernel (SwiGLU, bf16, 16-byte chunks, dense) on the",
        "# glu_qwen3_4b workload (16384 x 9728): forward reads e, g and writes h;",
        "# backward reads dh, e, g and writes de, dg.",
        "# Two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) over the same bench",
        "# command, each counter scaled by its reading for a plain 1 GiB device copy.",
        f"# commands: {command}",
    ]
    lines = []
    for name, per_elem in (("fwd", 3), ("bwd", 5)):
        m = _pmc_scaled(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv,
                        GLU_KERNEL_KEYS[name])
        lines += _pmc_lines(m, per_elem * w.elements * w.elem_bytes, prefix=f"{name}_")
    lines.append(f"kernel_source_sha256_16: {kernel_source_hash(GLU_SOURCES)}")
    _write_summary(GLU_TRAFFIC_FILE, header, lines)


COUNTERS_FILE = os.path.join(ROOT, "profiles", "rope_qk_cos_sin_fly_vs_table_counters.txt")
CU_COUNT, SIMDS_PER_CU, XCDS = 256, 4, 8


def _kernel_counters(run_dir: str) -> dict:
    """Mean per-dispatch value of every counter in the rocprofv3 --pmc CSVs under
    run_dir (one pass per subfolder), over the dispatches of the RoPE kernel."""
    import csv
    import glob
    acc = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if "rope_qk" in row["Kernel_Name"]:
                    acc.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _kernel_durations_us(run_dir: str) -> np.ndarray:
    import csv
    import glob
    d = []
    for path in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if "rope_qk" in row["Kernel_Name"]:
                    d.append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    return np.array(d)


def write_counters_summary(fly_dir, table_dir, copy_fetch_csv, copy_write_csv, command):
    """Counters of the row-group kernel on the Qwen3-4B batch with cos/sin evaluated in
    the kernel (fly) and read from a cos/sin cache (table): instruction mix per wave,
    VALU issue, wave lifetime, HBM bytes (scaled by a 1 GiB device copy's readings)
    and per-launch time from kernel traces of the same commands."""
    w = workloads.get("qwen3_4b_packed")
    bpl = algorithmic_bytes_per_launch(w)
    copy_bytes = 2 ** 30
    f_c = max(v[0] for v in _dispatch_means(copy_fetch_csv).values())
    w_c = max(v[0] for v in _dispatch_means(copy_write_csv).values())
    f_scale, w_scale = copy_bytes / (f_c * 1024.0), copy_bytes / (w_c * 1024.0)
    runs = {"fly": _kernel_counters(fly_dir), "table": _kernel_counters(table_dir)}
    times = {"fly": _kernel_durations_us(fly_dir), "table": _kernel_durations_us(table_dir)}
    simds = CU_COUNT * SIMDS_PER_CU

    def row(name, fn, fmt="{:.4g}"):
        vals = {m: fn(runs[m], times[m]) for m in runs}
        ratio = vals["table"] / vals["fly"] if vals["fly"] else float("nan")
        return f"{name:44s} {fmt.format(vals['fly']):>14s} {fmt.format(vals['table']):>14s}   x{ratio:.3f}"

    per_wave = lambda k: (lambda c, t: c[k] / c["SQ_WAVES"])
    lines = [
        f"{'quantity (per launch of the RoPE kernel)':44s} {'fly':>14s} {'table':>14s}   table/fly",
        row("kernel duration, kernel trace (us)", lambda c, t: float(t.mean()), "{:.2f}"),
        row("waves (SQ_WAVES)", lambda c, t: c["SQ_WAVES"], "{:.0f}"),
        row("VALU instructions per wave", per_wave("SQ_INSTS_VALU"), "{:.1f}"),
        row("  of which fp64 FMA", per_wave("SQ_INSTS_VALU_FMA_F64"), "{:.1f}"),
        row("SALU instructions per wave", per_wave("SQ_INSTS_SALU"), "{:.1f}"),
        row("scalar memory instructions per wave", per_wave("SQ_INSTS_SMEM"), "{:.1f}"),
        row("LDS instructions per wave", per_wave("SQ_INSTS_LDS"), "{:.1f}"),
        row("vector memory reads per wave", per_wave("SQ_INSTS_VMEM_RD"), "{:.1f}"),
        row("vector memory writes per wave", per_wave("SQ_INSTS_VMEM_WR"), "{:.1f}"),
        row("LDS bank conflict cycles", lambda c, t: c["SQ_LDS_BANK_CONFLICT"], "{:.0f}"),
        row("VALU busy, % of SIMD issue cycles",
            lambda c, t: 100.0 * 4 * c["SQ_ACTIVE_INST_VALU"] / (simds * c["GRBM_GUI_ACTIVE"] / XCDS),
            "{:.1f}"),
        row("wave lifetime (SQ_WAVE_CYCLES / SQ_WAVES)", per_wave("SQ_WAVE_CYCLES"), "{:.0f}"),
        row("cycles waiting per wave (SQ_WAIT_INST_ANY)", per_wave("SQ_WAIT_INST_ANY"), "{:.0f}"),
    ]
    if all("TA_TA_BUSY_sum" in runs[m] for m in runs):
        per_cu = lambda k: (lambda c, t: 100.0 * c[k] / (CU_COUNT * c["GRBM_GUI_ACTIVE"] / XCDS))
        lines += [
            row("TA busy, % of cycles per CU", per_cu("TA_TA_BUSY_sum"), "{:.1f}"),
            row("TD busy, % of cycles per CU", per_cu("TD_TD_BUSY_sum"), "{:.1f}"),
            row("TA stalled by the cache, % of cycles",
                per_cu("TA_DATA_STALLED_BY_TC_CYCLES_sum"), "{:.1f}"),
            row("TCP stalled on pending data, % of cycles",
                per_cu("TCP_PENDING_STALL_CYCLES_sum"), "{:.1f}"),
            row("L2 read latency seen by TCP (cycles/request)",
                lambda c, t: c["TCP_TCC_READ_REQ_LATENCY_sum"] / c["TCP_TCC_READ_REQ_sum"],
                "{:.0f}"),
        ]
    lines += [
        row("HBM read bytes (FETCH_SIZE x scale)",
            lambda c, t: c["FETCH_SIZE"] * 1024.0 * f_scale, "{:.4g}"),
        row("HBM write bytes (WRITE_SIZE x scale)",
            lambda c, t: c["WRITE_SIZE"] * 1024.0 * w_scale, "{:.4g}"),
        f"algorithmic bytes per launch: {bpl} (one read + one write of Q and K)",
        f"FETCH_SIZE scale {f_scale:.5f}, WRITE_SIZE scale {w_scale:.5f} (1 GiB device copy)",
    ]
    header = [
        "# cos/sin in the kernel (fly) versus from a cos/sin cache (table): counters of the",
        "# row-group kernel on the qwen3_4b_packed workload (T=16384, Hq=32, Hkv=8, D=128,",
        "# bf16, theta=1e6). Both give bit-identical results (the cache is written by the",
        "# library's own cos/sin export). Counter values are per dispatch, summed over the",
        "# chip; VALU busy takes 4 cycles per wave64 VALU instruction (SQ_ACTIVE_INST_VALU",
        "# counts instructions issued) against 1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs cycles.",
        f"# commands (R = repository root, M = fly or table): {command}",
        "",
    ]
    _write_summary(COUNTERS_FILE, header, lines)


PADDED_COUNTERS_FILE = os.path.join(ROOT, "profiles", "rope_qk_qwen3_8b_padded_counters.txt")


def write_padded_counters_summary(padded_dir, packed_dir, copy_fetch_csv, copy_write_csv,
                                  command):
    """Counters of the padded layout's seqused launch (token kernel, 8 x 2048 rows)
    beside the packed batch of the same sequences (row-group kernel): waves, their
    lifetime and instruction mix, memory-unit busy, HBM bytes (scaled by a 1 GiB copy's
    readings) and kernel-trace durations, per dispatch."""
    wp, wk = workloads.get("qwen3_8b_padded"), workloads.get("qwen3_8b_packed")
    bpl = algorithmic_bytes_per_launch(wp)
    copy_bytes = 2 ** 30
    f_c = max(v[0] for v in _dispatch_means(copy_fetch_csv).values())
    w_c = max(v[0] for v in _dispatch_means(copy_write_csv).values())
    f_scale, w_scale = copy_bytes / (f_c * 1024.0), copy_bytes / (w_c * 1024.0)
    runs = {"padded": _kernel_counters(padded_dir), "packed": _kernel_counters(packed_dir)}
    times = {"padded": _kernel_durations_us(padded_dir), "packed": _kernel_durations_us(packed_dir)}

    def row(name, fn, fmt="{:.4g}"):
        vals = {m: fn(runs[m], times[m]) for m in runs}
        ratio = vals["padded"] / vals["packed"] if vals["packed"] else float("nan")
        return (f"{name:46s} {fmt.format(vals['padded']):>12s} {fmt.format(vals['packed']):>12s}"
                f"   x{ratio:.3f}")

    per_wave = lambda k: (lambda c, t: c[k] / c["SQ_WAVES"])
    per_cu = lambda k: (lambda c, t: 100.0 * c[k] / (CU_COUNT * c["GRBM_GUI_ACTIVE"] / XCDS))
    lines = [
        f"{'quantity (per launch)':46s} {'padded':>12s} {'packed':>12s}   padded/packed",
        row("kernel duration, kernel trace (us)", lambda c, t: float(t.mean()), "{:.2f}"),
        row("waves (SQ_WAVES)", lambda c, t: c["SQ_WAVES"], "{:.0f}"),
        row("wave lifetime, cycles (SQ_WAVE_CYCLES/SQ_WAVES)", per_wave("SQ_WAVE_CYCLES"), "{:.0f}"),
        row("wave-cycles in all waves (SQ_WAVE_CYCLES)", lambda c, t: c["SQ_WAVE_CYCLES"], "{:.4g}"),
        row("VALU instructions per wave", per_wave("SQ_INSTS_VALU"), "{:.1f}"),
        row("scalar memory instructions per wave", per_wave("SQ_INSTS_SMEM"), "{:.1f}"),
        row("vector memory reads per wave", per_wave("SQ_INSTS_VMEM_RD"), "{:.1f}"),
        row("vector memory writes per wave", per_wave("SQ_INSTS_VMEM_WR"), "{:.1f}"),
        row("cycles waiting per wave (SQ_WAIT_INST_ANY)", per_wave("SQ_WAIT_INST_ANY"), "{:.0f}"),
        row("TA busy, % of cycles per CU", per_cu("TA_TA_BUSY_sum"), "{:.1f}"),
        row("TA stalled by the cache, % of cycles", per_cu("TA_DATA_STALLED_BY_TC_CYCLES_sum"),
            "{:.1f}"),
        row("HBM read bytes (FETCH_SIZE x scale)",
            lambda c, t: c["FETCH_SIZE"] * 1024.0 * f_scale, "{:.4g}"),
        row("HBM write bytes (WRITE_SIZE x scale)",
            lambda c, t: c["WRITE_SIZE"] * 1024.0 * w_scale, "{:.4g}"),
        f"algorithmic bytes per launch (valid tokens only): {bpl} for both; rows: padded "
        f"{wp.T}, packed {wk.T} ({wp.valid_tokens} valid)",
        f"FETCH_SIZE scale {f_scale:.5f}, WRITE_SIZE scale {w_scale:.5f} (1 GiB device copy)",
    ]
    header = [
        "# The padded layout: the same 8 sequences (lengths U{256..2048}, Hq=32, Hkv=8, D=128,",
        "# bf16) as 8 x 2048 rows through the seqused launch of the plain entry point (padded",
        "# rows skipped; the token kernel, one wave per token) and packed (row-group kernel, 5",
        "# waves per token). rocprofv3 --pmc passes (per-dispatch means, summed over the chip)",
        "# and a kernel trace of each command.",
        f"# commands (R = repository root, W = qwen3_8b_padded or qwen3_8b_packed): {command}",
        "",
    ]
    _write_summary(PADDED_COUNTERS_FILE, header, lines)


def trace_summary_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"rope_qk_{workload}_kernel_trace.txt")


def expected_grid_threads(w: workloads.Workload, padded: str = "compact") -> list:
    """Work-items of each launch of the default pass for this workload: one 64-lane
    workgroup per (token, row group) for the row-group kernel (per rotated token only,
    for a compact padded launch), one 64-lane wave per token for the token kernel."""
    if rope_kernel_name(w, 0, padded) == "rope_qk_group_kernel":
        rows = rows_per_workgroup(w)
        groups = -(-w.Hq // rows) + -(-w.Hkv // rows)
        return [t * groups * 64 for t in launch_pieces(w, padded)]
    return [w.T * 64]


def write_trace_summary(trace_csv: str, workload: str, command: str) -> None:
    """Per-launch durations of the RoPE kernel from a rocprofv3 --kernel-trace CSV
    (one row per dispatch), with the algorithmic bandwidth they give, as a small
    text summary under profiles/. Only the dispatches of this workload's default
    launch count (its kernel instance and grid size), so a trace of the default
    bench command, which runs every workload, serves each of them."""
    import csv
    w = workloads.get(workload)
    keys = rope_instance_names(w, needs_long_index(w))
    key = keys[0]
    grids = expected_grid_threads(w)
    pieces = len(grids)
    durs, names, shapes = [], set(), {}
    with open(trace_csv) as fh:
        for row in csv.DictReader(fh):
            if not any(k in row["Kernel_Name"] for k in keys) or \
                    int(row["Grid_Size_X"]) not in grids:
                continue
            durs.append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
            names.add(row["Kernel_Name"])
            shapes[row["Grid_Size_X"]] = (row["Grid_Size_X"], row["Workgroup_Size_X"],
                                          row["VGPR_Count"], row["LDS_Block_Size"])
    if not durs:
        raise SystemExit(f"no dispatch of {key} with {grids} work-items in {trace_csv}")
    d = np.array(durs)
    bpl = algorithmic_bytes_per_launch(w)

    def rate(us):
        gbps = bpl / (us * 1e-6) / 1e9
        return f"{us:.2f} us -> {gbps:.0f} GB/s = {100 * gbps / HBM_PEAK_GBPS:.1f}% of 8 TB/s"

    seq = "padded rows skipped via seqused" if w.seqused is not None else "packed"
    header = [
        f"# rocprofv3 kernel trace: RoPE kernel on the {w.name} workload",
        f"# (T={w.T} rows, {w.valid_tokens} valid tokens in {len(w.cu_seqlens) - 1} sequences, "
        f"{seq}; Hq={w.Hq}, Hkv={w.Hkv}, D={w.D}, {w.dtype}, theta={w.theta:g})",
        "# every timed step = forward(Q, K) + backward(dQ, dK), one launch each"
        + ("" if pieces == 1 else f" (here {pieces} launches each, over consecutive token ranges)")
        + ";",
        "# buffer sets rotate so that no launch is served from the Infinity Cache",
        f"# command (R = repository root, on one MI355X): {command}",
        "",
    ]
    lines = ["kernel: " + ", ".join(sorted(names))]
    lines += [f"grid_threads, workgroup, vgprs, static_lds_bytes: {', '.join(sh)}"
              for sh in shapes.values()]
    if any("group_kernel" in n for n in names):
        lines += ["(rocprofv3's LDS column is the kernel's static LDS only: the dynamic LDS the",
                  " row-group launch reserves to cap residency per CU is allocated but not shown)"]
    if pieces > 1:
        lines.append(f"launches_per_pass: {pieces} (tokens per launch: "
                     f"{', '.join(str(t) for t in sorted(set(launch_pieces(w))))})")
    lines += [
        f"dispatches: {len(d)} (warmup included)",
        f"algorithmic_bytes_per_launch: {bpl:.0f} (one read + one write of every rotated element"
        + ("" if pieces == 1 else f"; the pass's {algorithmic_bytes_per_pass(w)} over {pieces} launches")
        + ")",
        f"average: {rate(float(d.mean()))}",
        f"median:  {rate(float(np.median(d)))}",
        f"minimum: {rate(float(d.min()))}",
        f"maximum: {float(d.max()):.2f} us",
        f"valid_tokens_per_s_at_average: {w.valid_tokens / (pieces * float(d.mean()) * 1e-6):.4g} "
        "per pass (forward or backward)",
    ]
    _write_summary(trace_summary_path(workload), header, lines)


GLU_TRACE_FILE = os.path.join(ROOT, "profiles", "glu_qwen3_4b_kernel_trace.txt")
GLU_KIND_CODES = {"swiglu": 0, "geglu": 1, "geglu_tanh": 2}


def write_glu_trace_summary(run_dir: str, command: str) -> None:
    """Per-launch durations of glu_kernel (bf16, dense, 32-bit offsets) on glu_qwen3_4b
    for the three kinds, from run_dir/glu_trace_<kind>/*kernel_trace.csv (rocprofv3)
    beside each kind's bench.py JSON line in run_dir/glu_bench_<kind>.log."""
    import csv
    import glob
    w = workloads.glu_get("glu_qwen3_4b")
    per = {"forward": 3 * w.elements * w.elem_bytes, "backward": 5 * w.elements * w.elem_bytes}
    lines = [f"{'kind':11s} {'launch':9s} {'calls':>5s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s}"
             f"  {'avg GB/s (% of 8 TB/s)':24s} bench.py events avg_us (GB/s)"]
    for kind, code in GLU_KIND_CODES.items():
        durs = {"forward": [], "backward": []}
        for path in glob.glob(os.path.join(run_dir, f"glu_trace_{kind}", "**", "*kernel_trace.csv"),
                              recursive=True):
            with open(path) as fh:
                for row in csv.DictReader(fh):
                    name = row["Kernel_Name"]
                    for launch, bwd in (("forward", 0), ("backward", 1)):
                        if glu_instance(code, bwd) in name:
                            durs[launch].append((int(row["End_Timestamp"])
                                                 - int(row["Start_Timestamp"])) / 1e3)
        with open(os.path.join(run_dir, f"glu_bench_{kind}.log")) as fh:
            js = json.loads([ln for ln in fh if ln.startswith("{")][-1])
        ev = {"forward": js["forward"]["avg_launch_us"], "backward": js["roofline"]["avg_launch_us"]}
        for launch in ("forward", "backward"):
            d = np.array(durs[launch])
            if d.size == 0:
                raise SystemExit(f"no {kind} {launch} dispatch under {run_dir}")
            gbps = per[launch] / (d.mean() * 1e-6) / 1e9
            egbps = per[launch] / (ev[launch] * 1e-6) / 1e9
            lines.append(f"{kind:11s} {launch:9s} {d.size:5d} {d.mean():8.2f} {d.min():8.2f} "
                         f"{d.max():8.2f}  {gbps:6.0f} ({100 * gbps / HBM_PEAK_GBPS:4.1f}%)"
                         f"{'':12s} {ev[launch]:.2f} ({egbps:.0f})")
    header = [
        "# rocprofv3 kernel traces: glu_kernel on the glu_qwen3_4b workload (16384 tokens x 9728,",
        "# the Qwen3-4B MLP width, bf16, N(0,1) e, g, dh; forward (e, g -> h) + backward",
        "# (dh, e, g -> de, dg) per step, 2 rotating buffer sets of 1.9 GB)",
        f"# commands (R = repository root, on one MI355X), for K in swiglu geglu geglu_tanh: {command}",
        f"# algorithmic bytes per launch: forward {per['forward']} (read e, g; write h),",
        f"#                               backward {per['backward']} (read dh, e, g; write de, dg)",
        "# Instances: glu_kernel<__bf16, VEC=8, KIND, BWD, DENSE=true, uint32 offsets (int64 for the",
        "# tanh-GeGLU backward, the library's default there)>; the other",
        "# kernels in the traces are torch's input generation and copies (not timed).",
        "",
    ]
    _write_summary(GLU_TRACE_FILE, header, lines)


GLU_VALU_FILE = os.path.join(ROOT, "profiles", "glu_valu_occupancy.txt")


def write_glu_valu_summary(run_dir: str, command: str) -> None:
    """VALU occupancy of glu_kernel's forward and backward for the three kinds, from one
    rocprofv3 --pmc pass each (run_dir/<kind>/*counter_collection.csv)."""
    import glob
    lines = [f"{'kind':12s} {'pass':8s} {'waves':>8s} {'VALU instr/wave':>16s} {'VALU busy':>10s}"
             f" {'GRBM cycles/XCD':>16s}"]
    simds = CU_COUNT * SIMDS_PER_CU
    for kind, code in GLU_KIND_CODES.items():
        for launch, bwd in (("forward", 0), ("backward", 1)):
            acc = {}
            for path in glob.glob(os.path.join(run_dir, kind, "**", "*counter_collection.csv"),
                                  recursive=True):
                with open(path) as fh:
                    for row in csv.DictReader(fh):
                        if glu_instance(code, bwd) in row["Kernel_Name"]:
                            acc.setdefault(row["Counter_Name"], []).append(
                                float(row["Counter_Value"]))
            m = {k: sum(v) / len(v) for k, v in acc.items()}
            busy = 100.0 * 4 * m["SQ_ACTIVE_INST_VALU"] / (simds * m["GRBM_GUI_ACTIVE"] / XCDS)
            lines.append(f"{kind:12s} {launch:8s} {m['SQ_WAVES']:8.0f} "
                         f"{m['SQ_INSTS_VALU'] / m['SQ_WAVES']:16.0f} {busy:9.1f}% "
                         f"{m['GRBM_GUI_ACTIVE'] / XCDS:16.0f}")
    header = [
        "# VALU occupancy of glu_kernel on the glu_qwen3_4b workload (16384 x 9728 bf16), one",
        "# rocprofv3 --pmc pass per kind; per-dispatch means over the forward and the backward",
        "# dispatches. VALU busy = SQ_ACTIVE_INST_VALU x 4 cycles / (1024 SIMDs x",
        "# GRBM_GUI_ACTIVE / 8 XCDs).",
        f"# command (R = repository root, on one MI355X), for K in swiglu geglu geglu_tanh: {command}",
        "",
    ]
    _write_summary(GLU_VALU_FILE, header, lines)


def packed_position_ids(w: workloads.Workload) -> np.ndarray:
    """Per-token positions of the packed batch (0..len-1 per sequence; -1 for rows
    outside every sequence): the position_ids a 1-D packing collator would emit."""
    ids = np.full(w.T, -1, dtype=np.int32)
    for s0, n in zip(w.cu_seqlens[:-1], w.lengths):
        ids[s0:s0 + n] = np.arange(n, dtype=np.int32)
    return ids


def make_sets(w, nsets, dev, layout="contiguous"):
    """nsets independent buffer sets {q, k, dq, dk}. With layout "qkv" the four are
    [T, H, D] views into fused projection outputs [T, (Hq + 2 Hkv) D] (and their
    gradients), as a model's QKV projection produces them; V stays untouched."""
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    su = None if w.seqused is None else torch.from_numpy(w.seqused).to(dev)
    sets = []
    for i in range(nsets):
        if layout == "qkv":
            s = {}
            for fwd, grad in (("q", "k"), ("dq", "dk")):
                buf = workloads.make_tensor((w.T, (w.Hq + 2 * w.Hkv) * w.D),
                                            w.seed(fwd) + 100 * i, w.dtype, device=dev,
                                            chunk_rows=65536)
                s[fwd] = buf[:, :w.Hq * w.D].view(w.T, w.Hq, w.D)
                s[grad] = buf[:, w.Hq * w.D:(w.Hq + w.Hkv) * w.D].view(w.T, w.Hkv, w.D)
            sets.append(s)
            continue
        sets.append({what: workloads.make_tensor(w.shape(what), w.seed(what) + 100 * i, w.dtype,
                                                 device=dev, chunk_rows=65536)
                     for what in ("q", "k", "dq", "dk")})
    return cu, su, sets


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed_reps(fn, budget_s: float, cap: int):
    total, reps = 0.0, 0
    while total < budget_s and reps < cap:
        total += fn()
        reps += 1
    return reps, total


def cpu_baseline(w, budget_s: float, nthreads: int):
    """The oracle, as it stands, on the same workload: whole fwd+bwd passes over the
    batch, repeated until about budget_s seconds of work have been timed on
    nthreads host threads, then a quarter of that on one thread."""
    import oracle

    host = {what: workloads.host_bits(workloads.make_tensor(w.shape(what), w.seed(what), w.dtype))
            for what in ("q", "k", "dq", "dk")}

    def one(threads):
        return lambda: oracle.fwd_bwd_seconds(host["q"], host["k"], host["dq"], host["dk"],
                                              w.cu_seqlens, w.theta, w.dtype, w.seqused, threads)

    reps, total = _timed_reps(one(nthreads), budget_s, 10000)
    reps1, total1 = _timed_reps(one(1), budget_s / 4, 10000)
    step_bytes = 2 * algorithmic_bytes_per_pass(w)  # the GPU's byte count for fwd + bwd
    return {
        "value": w.valid_tokens * reps / total,
        "unit": "tokens/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": f"{reps} full fwd+bwd passes over the {w.name} batch "
                  f"({w.valid_tokens} tokens, Q/K/dQ/dK), {total:.1f} s timed",
        "seconds_per_pass_pair": total / reps,
        "GBps": step_bytes * reps / total / 1e9,
        "value_1_core": w.valid_tokens * reps1 / total1,
        "GBps_1_core": step_bytes * reps1 / total1 / 1e9,
        "cpu_model": cpu_model(),
    }


def copy_calibration(gib: float, reps: int):
    """A plain device copy of known size, for scaling PMC byte counters."""
    n = int(gib * 2 ** 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "reps": reps}))


def compare_unfused(rope, w, cu, su, sets, nsets, args, stream):
    """Fused in-place QK-RoPE against unfused variants built from the same kernel, on
    the same buffers: one step = forward on (Q, K) + backward on (dQ, dK).
      fused            one launch per pass, in place (the library's path)
      separate         Q and K in two launches per pass, in place
      separate_clone   clone Q and K (out-of-place result), two launches on the clones
      transpose_clone  per tensor: contiguous transpose to [H, T, D], rotate with
                       explicit per-row positions, contiguous transpose back
    Prints one JSON line with per-step times and ratios to fused."""
    dev = sets[0]["q"].device
    empty = {}

    def no_heads(x, like):
        key = (x, like.dtype)
        if key not in empty:
            empty[key] = torch.empty((w.T, 0, w.D), dtype=like.dtype, device=dev)
        return empty[key]

    ids_np = packed_position_ids(w)
    ids_by_h = {}

    def head_major_ids(H):
        if H not in ids_by_h:
            ids_by_h[H] = torch.from_numpy(np.tile(ids_np, H)).to(dev)
        return ids_by_h[H]

    def fused(s, qn, kn, d):
        rope.qk_apply_(s[qn], s[kn], cu, w.theta, d, seqused=su)

    def separate(s, qn, kn, d):
        rope.qk_apply_(s[qn], no_heads("k", s[kn]), cu, w.theta, d, seqused=su)
        rope.qk_apply_(no_heads("q", s[qn]), s[kn], cu, w.theta, d, seqused=su)

    def separate_clone(s, qn, kn, d):
        q2 = s[qn].clone()
        rope.qk_apply_(q2, no_heads("k", q2), cu, w.theta, d, seqused=su)
        k2 = s[kn].clone()
        rope.qk_apply_(no_heads("q", k2), k2, cu, w.theta, d, seqused=su)
        return q2, k2

    def transpose_clone(s, qn, kn, d):
        out = []
        for name in (qn, kn):
            x = s[name]
            H = x.shape[1]
            xt = x.transpose(0, 1).contiguous().view(H * w.T, 1, w.D)
            rope.qk_apply_ex_(xt, torch.empty((H * w.T, 0, w.D), dtype=x.dtype, device=dev),
                              w.theta, d, position_ids=head_major_ids(H))
            out.append(xt.view(H, w.T, w.D).transpose(0, 1).contiguous())
        return out

    variants = {"fused": fused, "separate": separate, "separate_clone": separate_clone,
                "transpose_clone": transpose_clone}
    res = {}
    for name, fn in variants.items():
        def step(i):
            s = sets[i % nsets]
            fn(s, "q", "k", 1)
            fn(s, "dq", "dk", -1)
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) / args.steps * 1e6
    out = {
        "compare": "fused in-place QK-RoPE vs unfused variants (fwd+bwd step)",
        "workload": w.name, "T": w.T, "valid_tokens": w.valid_tokens, "Hq": w.Hq, "Hkv": w.Hkv,
        "D": w.D, "dtype": w.dtype, "steps": args.steps,
        "us_per_step": {k: round(v, 2) for k, v in res.items()},
        "speedup_of_fused": {k: round(v / res["fused"], 3) for k, v in res.items()},
    }
    print(json.dumps(out))


def rope_kernel_instance(w: workloads.Workload, long_index: bool, padded: str = "compact") -> str:
    """Mangled-name fragment of the default path's kernel instance for this workload
    (kernel, dtype, chunk width, index width, no tables, and for the row-group kernel
    whether the launch is compact, whether it is staged and its row steps), as
    rocprofv3 lists it."""
    base = rope_kernel_name(w, 0, padded)
    dt = {"bf16": "DF16b", "f16": "DF16_", "f32": "f"}[w.dtype]
    vec = chunk_bytes(w) // w.elem_bytes
    name = f"{base}I{dt}Li{vec}ELb{int(long_index)}ELb0E"
    if base == "rope_qk_group_kernel":
        name += (f"Lb{int(compact_launch(w, padded))}ELb{int(staged_geometry(w))}E"
                 f"Li{group_steps(w)}E")
    return name


def rope_instance_names(w: workloads.Workload, long_index: bool, padded: str = "compact") -> tuple:
    """The instance's name as rocprofv3 may list it: mangled, or demangled."""
    base = rope_kernel_name(w, 0, padded)
    dt = {"bf16": "__bf16", "f16": "_Float16", "f32": "float"}[w.dtype]
    vec = chunk_bytes(w) // w.elem_bytes
    flags = [str(long_index).lower(), "false"]
    if base == "rope_qk_group_kernel":
        flags.append(str(compact_launch(w, padded)).lower())
        flags.append(str(staged_geometry(w)).lower())
        flags.append(str(group_steps(w)))
    demangled = f"{base}<{dt}, {vec}, {', '.join(flags)}>"
    return rope_kernel_instance(w, long_index, padded), demangled


def needs_long_index(w: workloads.Workload) -> bool:
    return w.T * (w.Hq + w.Hkv) * w.D >= 2 ** 31


def region_us(stream: int, launches, n: int) -> float:
    """Average GPU time per call of launches(i) over n back-to-back calls, from one
    pair of HIP events on the launch stream (gaps between launches included)."""
    ev = [HipEvent(), HipEvent()]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        launches(i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_ms(ev[1]) * 1e3 / n


def inplace_reference_us(sets, nsets, stream, n: int) -> float:
    """Per-pass time of a torch in-place elementwise op over the same bytes as one
    RoPE launch: negate Q, then K (two launches, each one read and one write of its
    tensor), on the same rotating buffer sets."""
    def one(i):
        s = sets[i % nsets]
        s["q"].neg_()
        s["k"].neg_()
    for i in range(min(n, 2 * nsets)):
        one(i)
    return region_us(stream, one, n)


def padded_metadata(rope, w: workloads.Workload, cu, su):
    """cu_valid (the library's prefix kernel, once per batch, as a trainer builds it
    beside cu_seqlens) and the host count of rotated tokens of a padded workload."""
    return rope.valid_prefix(cu, su), w.valid_tokens


def time_workload(rope, w: workloads.Workload, dev, n_steps: int, warmup: int,
                  min_warmup_s: float = 0.05, min_timed_s: float = 0.1,
                  padded: str = "compact") -> dict:
    """Region-timed default launches (forward + backward per step) of one workload on
    its own rotating buffer sets, beside the torch in-place reference over the same
    bytes (fully packed workloads only: a padded layout's valid bytes are not one
    tensor). Warm-up runs at least `warmup` steps and `min_warmup_s` seconds (the
    GPU's clocks settle after the previous workload), the timed region at least
    `n_steps` steps and `min_timed_s` seconds. A padded workload is launched compact
    (padded == "compact") and, for comparison, also timed through the seqused launch
    of the plain entry point."""
    set_bytes = 2 * w.T * (w.Hq + w.Hkv) * w.D * w.elem_bytes
    nsets = max(2, math.ceil(8 * INFINITY_CACHE_BYTES / set_bytes))
    cu, su, sets = make_sets(w, nsets, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    compact = compact_launch(w, padded)
    if compact:
        cv, valid = padded_metadata(rope, w, cu, su)

    def step_compact(i):
        s = sets[i % nsets]
        rope.qk_apply_padded_(s["q"], s["k"], w.theta, 1, cu, su, cv, valid)
        rope.qk_apply_padded_(s["dq"], s["dk"], w.theta, -1, cu, su, cv, valid)

    def step_plain(i):
        s = sets[i % nsets]
        rope.qk_apply_(s["q"], s["k"], cu, w.theta, 1, seqused=su)
        rope.qk_apply_(s["dq"], s["dk"], cu, w.theta, -1, seqused=su)

    def timed(step):
        step_us = region_us(stream, step, 10)
        for i in range(max(warmup, math.ceil(min_warmup_s * 1e6 / step_us))):
            step(i)
        n = max(n_steps, math.ceil(min_timed_s * 1e6 / step_us))
        return region_us(stream, step, n) / 2, n

    pass_us, n_steps = timed(step_compact if compact else step_plain)
    pieces = len(launch_pieces(w, padded))
    bpp = algorithmic_bytes_per_pass(w)
    gbps = bpp / (pass_us * 1e-6) / 1e9
    out = {
        "T": w.T, "valid_tokens": w.valid_tokens, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
        "dtype": w.dtype, "kernel": rope_kernel_name(w, 0, padded),
        "index": "64-bit" if needs_long_index(w) else "32-bit",
        "launches_per_pass": pieces, "bytes_per_launch": bpp / pieces,
        "avg_launch_us": pass_us / pieces, "avg_pass_us": pass_us, "GBps": gbps,
        "frac": gbps / HBM_PEAK_GBPS,
        "fwd_bwd_tokens_per_s": w.valid_tokens / (2 * pass_us * 1e-6),
        "passes_timed": 2 * n_steps,
    }
    if w.seqused is not None:
        out["padded_launch"] = padded
        if compact:
            plain_us, _ = timed(step_plain)
            out["seqused_launch_us"] = plain_us
            out["seqused_kernel"] = rope_kernel_name(w, 0, "seqused")
            out["seqused_frac"] = bpp / (plain_us * 1e-6) / 1e9 / HBM_PEAK_GBPS
    if w.seqused is None:
        ref_us = inplace_reference_us(sets, nsets, stream, 2 * n_steps)
        out["torch_inplace_us"] = ref_us
        out["torch_inplace_GBps"] = bpp / (ref_us * 1e-6) / 1e9
        out["frac_of_ceiling"] = ref_us / pass_us
    del sets
    torch.cuda.empty_cache()
    return out


def cpu_baseline_sampled(w: workloads.Workload, sets0: dict, budget_s: float, nthreads: int,
                         n_tokens: int = 1024) -> dict:
    """The oracle, as it stands, on evenly spaced tokens of a workload too large to
    process whole: their rows of Q, K, dQ and dK (copied from the benchmark's first
    buffer set, the same bits the GPU rotates) go through the oracle's forward and
    backward, repeated for about budget_s seconds on nthreads threads, then a
    quarter of that on one thread. tokens/s = sampled tokens per pass pair / time."""
    import oracle

    tokens = np.unique(np.linspace(0, w.T - 1, n_tokens).astype(np.int64))
    idx = torch.from_numpy(tokens).to(sets0["q"].device)
    rows = {what: workloads.host_bits(sets0[what].index_select(0, idx))
            for what in ("q", "k", "dq", "dk")}
    timer = oracle.rows_fwd_bwd_timer(rows["q"], rows["k"], rows["dq"], rows["dk"], tokens,
                                      w.cu_seqlens, w.theta, w.dtype, w.seqused)
    timer(nthreads)  # first touch of the output buffers, not timed
    reps, total = _timed_reps(lambda: timer(nthreads), budget_s, 100000)
    reps1, total1 = _timed_reps(lambda: timer(1), budget_s / 4, 100000)
    n = tokens.size
    tok_bytes = 2 * 2 * (w.Hq + w.Hkv) * w.D * w.elem_bytes  # the GPU's count, fwd + bwd
    return {
        "value": n * reps / total,
        "unit": "tokens/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": f"{n} evenly spaced tokens of the {w.name} workload (T={w.T}): their rows "
                  f"of Q, K, dQ, dK through the oracle's forward + backward, {reps} passes, "
                  f"{total:.1f} s timed",
        "seconds_per_token": total / (reps * n),
        "GBps": tok_bytes * n * reps / total / 1e9,
        "value_1_core": n * reps1 / total1,
        "GBps_1_core": tok_bytes * n * reps1 / total1 / 1e9,
        "cpu_model": cpu_model(),
    }


SWEEP_TOKENS = [2048, 4096, 8192, 8554, 12288, 16384, 24576, 32768, 65536, 131072, 262144,
                524288]
SWEEP_HEADS = (32, 8, 128)  # Hq, Hkv, D: the Qwen3-4B/8B attention shape
SWEEP_FILE = os.path.join(ROOT, "profiles", "rope_qk_size_sweep.txt")


def sweep_workload(T: int) -> workloads.Workload:
    """One sequence of T tokens in the 32 + 8 head, D = 128, bf16 shape."""
    Hq, Hkv, D = SWEEP_HEADS
    return workloads.Workload(f"sweep_{T}", 90, T, Hq, Hkv, D, "bf16", 1e6,
                              np.array([0, T], dtype=np.int32), description=f"one sequence, T={T}")


def linear_fit(x, y):
    """Least-squares t = t0 + b x; returns (t0, b)."""
    A = np.stack([np.ones(len(x)), np.asarray(x, dtype=np.float64)], 1)
    (t0, b), *_ = np.linalg.lstsq(A, np.asarray(y, dtype=np.float64), rcond=None)
    return float(t0), float(b)


def size_sweep(rope, dev, n_steps: int) -> dict:
    """Region-timed default launches and the torch in-place reference at every size
    of SWEEP_TOKENS, with t = t0 + b T fitted to each."""
    rows = []
    for T in SWEEP_TOKENS:
        print(f"[sweep] T={T}", file=sys.stderr, flush=True)
        r = time_workload(rope, sweep_workload(T), dev, n_steps, 20)
        rows.append({"T": T, "avg_pass_us": r["avg_pass_us"],
                     "launches_per_pass": r["launches_per_pass"],
                     "torch_inplace_us": r["torch_inplace_us"], "GBps": r["GBps"],
                     "index": r["index"]})
    per_token = 2 * (SWEEP_HEADS[0] + SWEEP_HEADS[1]) * SWEEP_HEADS[2] * 2
    out = {"sweep": "RoPE launch time vs tokens (one sequence, 32+8 heads, D=128, bf16)",
           "bytes_per_token": per_token, "rows": rows}
    for key in ("avg_pass_us", "torch_inplace_us"):
        t0, b = linear_fit([r["T"] for r in rows], [r[key] for r in rows])
        out[f"fit_{key}"] = {"t0_us": t0, "us_per_token": b,
                             "asymptotic_GBps": per_token / (b * 1e-6) / 1e9}
    return out


# Head shapes beside the Qwen3 batches: (Hq, Hkv, D, dtype), one sequence of
# HEAD_SHAPE_TOKENS tokens each. D = 128 with the Qwen3-1.7B (16 + 8), 4B/8B (32 + 8),
# 14B (40 + 8) and 32B (64 + 8) head counts; the staged head sizes (half rows that
# are not whole 128-byte lines, with one or two row steps), the long half rows
# D = 256 and 512, and the other storage types.
HEAD_SHAPES = [
    (16, 8, 128, "bf16"), (32, 8, 128, "bf16"), (40, 8, 128, "bf16"), (64, 8, 128, "bf16"),
    (32, 32, 32, "bf16"), (32, 32, 48, "bf16"), (32, 32, 64, "bf16"), (64, 8, 64, "bf16"),
    (32, 32, 80, "bf16"), (32, 32, 96, "bf16"), (32, 8, 96, "bf16"), (32, 32, 112, "bf16"),
    (32, 8, 112, "bf16"), (16, 16, 144, "bf16"), (16, 16, 160, "bf16"), (16, 16, 192, "bf16"),
    (16, 16, 176, "bf16"), (32, 8, 192, "bf16"), (16, 16, 224, "bf16"),
    (16, 16, 256, "bf16"), (16, 8, 256, "bf16"), (8, 8, 512, "bf16"),
    (32, 8, 128, "f16"), (32, 8, 128, "f32"), (32, 8, 64, "f32"),
]
HEAD_SHAPE_TOKENS = 16384
HEAD_SHAPES_FILE = os.path.join(ROOT, "profiles", "rope_qk_head_shapes.txt")


def head_shape_workload(Hq: int, Hkv: int, D: int, dtype: str,
                        T: int = HEAD_SHAPE_TOKENS) -> workloads.Workload:
    """One sequence of T tokens of the given head shape, theta = 1e6."""
    return workloads.Workload(f"h{Hq}x{Hkv}_d{D}_{dtype}", 92, T, Hq, Hkv, D, dtype, 1e6,
                              np.array([0, T], dtype=np.int32),
                              description=f"one sequence, T={T}, {Hq}+{Hkv} heads, D={D}")


def head_geometry(w: workloads.Workload) -> str:
    """The default launch's geometry for w: the row-group kernel (staged or not) with
    its rows per group, or the token kernel."""
    if rope_kernel_name(w, 0) != "rope_qk_group_kernel":
        return "token kernel"
    kind = "staged" if staged_geometry(w) else "row-group"
    steps = group_steps(w)
    if steps > 1 and staged_geometry(w):
        return f"{kind}, {rows_per_workgroup(w)} rows, 2 steps"
    rows = group_rows(chunks_per_half_row(w))
    return f"{kind}, {rows} rows" + (f" x {steps}" if steps > 1 else "")


def head_shape_survey(rope, dev, n_steps: int) -> dict:
    """Region-timed default launches (forward + backward per step, rotating buffer
    sets) and the torch in-place reference for every shape of HEAD_SHAPES."""
    rows = []
    for Hq, Hkv, D, dtype in HEAD_SHAPES:
        w = head_shape_workload(Hq, Hkv, D, dtype)
        print(f"[head shapes] {w.name}", file=sys.stderr, flush=True)
        r = time_workload(rope, w, dev, n_steps, 20)
        rows.append({"Hq": Hq, "Hkv": Hkv, "D": D, "dtype": dtype, "T": w.T,
                     "geometry": head_geometry(w), "launches_per_pass": r["launches_per_pass"],
                     "avg_pass_us": r["avg_pass_us"], "GBps": r["GBps"], "frac": r["frac"],
                     "torch_inplace_us": r["torch_inplace_us"],
                     "frac_of_ceiling": r["frac_of_ceiling"]})
    return {"head_shapes": f"RoPE pass per head shape (one sequence of {HEAD_SHAPE_TOKENS} "
                           "tokens, theta=1e6)", "rows": rows}


def write_head_shapes_summary(json_path: str, command: str) -> None:
    """profiles/rope_qk_head_shapes.txt from the JSON line of bench.py --head-shapes."""
    with open(json_path) as fh:
        js = json.loads([ln for ln in fh if ln.startswith("{")][-1])
    lines = [f"{'heads':>7s} {'D':>4s} {'dtype':>5s} {'geometry':>24s} {'launches':>8s} "
             f"{'pass us':>9s} {'GB/s':>6s} {'% peak':>7s} {'torch neg_ us':>14s} {'ratio':>6s}"]
    for r in js["rows"]:
        lines.append(f"{str(r['Hq']) + '+' + str(r['Hkv']):>7s} {r['D']:4d} {r['dtype']:>5s} "
                     f"{r['geometry']:>24s} {r['launches_per_pass']:8d} {r['avg_pass_us']:9.2f} "
                     f"{r['GBps']:6.0f} {100 * r['frac']:6.1f}% {r['torch_inplace_us']:14.2f} "
                     f"{r['frac_of_ceiling']:6.3f}")
    text = "\n".join([
        "# RoPE pass (one forward or backward launch set) per head shape on one MI355X:",
        f"# {js['head_shapes']}.",
        "# bench.py region timing (HIP events over back-to-back forward + backward steps",
        "# on rotating buffer sets that exceed the Infinity Cache),",
        "# GB/s = one read + one write of every Q and K element / pass time. 'torch neg_ us':",
        "# torch's in-place negation of the same Q and K tensors (two launches), the same",
        "# bytes through a bare elementwise kernel; ratio = its time / the RoPE pass time.",
        "# geometry: the default launch's kernel (staged: half rows that are not whole",
        "# 128-byte lines, moved through LDS) and its head rows per workgroup.",
        f"# command (R = repository root, on one MI355X): {command}",
        f"# kernel_source_sha256_16: {kernel_source_hash()}",
        "",
        *lines, ""])
    with open(HEAD_SHAPES_FILE, "w") as fh:
        fh.write(text)
    print(text)


def write_sweep_summary(run_dir: str, command: str) -> None:
    """profiles/rope_qk_size_sweep.txt from a rocprofv3 --kernel-trace of bench.py
    --sweep (run_dir/**/*kernel_trace.csv) and that run's JSON line
    (run_dir/sweep.json): per size, the RoPE pass's average duration from the trace
    (the sum of its launches' durations where a pass is several launches) and from
    region timing, torch's in-place reference (region timing), and t = t0 + b T
    fitted to each. The sizes run one after another, each one contiguous run of RoPE
    dispatches between torch's own kernels, which is how the trace is split."""
    import glob
    with open(os.path.join(run_dir, "sweep.json")) as fh:
        js = json.loads([ln for ln in fh if ln.startswith("{")][-1])
    events = []
    for path in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                events.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"]),
                               "rope_qk_group_kernel" in row["Kernel_Name"]))
    runs, cur = [], []
    for start, end, is_rope in sorted(events):
        if is_rope:
            cur.append((end - start) / 1e3)
        elif cur:
            runs.append(cur)
            cur = []
    if cur:
        runs.append(cur)
    if len(runs) != len(js["rows"]):
        raise SystemExit(f"{len(runs)} runs of RoPE dispatches for {len(js['rows'])} sizes")
    per_token = js["bytes_per_token"]
    lines = [f"{'tokens':>8s} {'launches':>8s} {'trace avg us':>13s} {'GB/s':>6s} {'% peak':>7s} "
             f"{'region us':>10s} {'torch neg_ us':>14s} {'torch GB/s':>10s} {'ratio':>6s} index"]
    xs, ys = [], []
    for r, run in zip(js["rows"], runs):
        T, n = r["T"], r["launches_per_pass"]
        if len(run) % n:
            raise SystemExit(f"T={T}: {len(run)} dispatches, not whole passes of {n}")
        avg = float(np.mean(np.array(run).reshape(-1, n).sum(1)))
        gb = per_token * T / (avg * 1e-6) / 1e9
        tgb = per_token * T / (r["torch_inplace_us"] * 1e-6) / 1e9
        lines.append(f"{T:8d} {n:8d} {avg:13.2f} {gb:6.0f} {100 * gb / HBM_PEAK_GBPS:6.1f}% "
                     f"{r['avg_pass_us']:10.2f} {r['torch_inplace_us']:14.2f} {tgb:10.0f} "
                     f"{r['torch_inplace_us'] / avg:6.3f} {r['index']}")
        if np.isfinite(avg):
            xs.append(T)
            ys.append(avg)
    def fit_line(label, x, y):
        t0, b = linear_fit(x, y)
        gb = per_token / (b * 1e-6) / 1e9
        return t0, b, (f"fit, {label}: t = {t0:.2f} us + T x {b * 1e3:.4f} ns -> incremental "
                       f"{gb:.0f} GB/s ({100 * gb / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")

    small = [i for i, T in enumerate(xs) if T <= 65536]
    torch_small = [r for r in js["rows"] if r["T"] <= 65536]
    t0, b, l_all = fit_line("RoPE kernel, trace averages, all sizes", xs, ys)
    t0s, bs, l_small = fit_line("RoPE kernel, trace averages, T <= 65536",
                                [xs[i] for i in small], [ys[i] for i in small])
    _, _, l_torch = fit_line("torch in-place neg_ on Q and K (two launches), T <= 65536",
                             [r["T"] for r in torch_small],
                             [r["torch_inplace_us"] for r in torch_small])
    lines += ["", l_all, l_small, l_torch]
    for T in (8554, 16384):
        t = t0s + bs * T
        lines.append(f"at T={T} (T <= 65536 fit): t = {t:.2f} us, of which the fixed part t0 is "
                     f"{t0s:.2f} us ({100 * t0s / t:.1f}%); without it the launch would take "
                     f"{bs * T:.2f} us = {100 * per_token * T / (bs * T * 1e-6) / 1e9 / HBM_PEAK_GBPS:.1f}%"
                     f" of 8 TB/s")
    header = [
        "# RoPE launch time against token count: one sequence of T tokens, Hq=32, Hkv=8, D=128,",
        "# bf16, theta=1e6, default launch (row-group kernel; 64-bit offsets at T=524288; a pass",
        "# of 2 x 327680 workgroups or more issued as launches over consecutive token ranges), each",
        "# size on its own rotating buffer sets (>= 2 GiB between touches of one buffer); beside",
        "# it torch's in-place neg_ over the same bytes (Q then K), the achievable-pattern reference.",
        f"# algorithmic bytes per token and launch: {per_token}",
        f"# command (R = repository root, on one MI355X): {command}",
        "",
    ]
    _write_summary(SWEEP_FILE, header, lines)


GLU_METRIC = "SwiGLU/GeGLU fwd+bwd tokens/s and achieved HBM GB/s (% of peak)"


def compare_glu_unfused(rope, w, kind, sets, nsets, args) -> None:
    """The library's fused GLU kernels against the same math as PyTorch eager ops
    (activation, product, and autograd for the backward), on the same buffers:
    wall time per forward and per backward. Context only: the unfused form moves
    intermediates through HBM."""
    act = {"swiglu": torch.nn.functional.silu,
           "geglu": lambda x: torch.nn.functional.gelu(x, approximate="none"),
           "geglu_tanh": lambda x: torch.nn.functional.gelu(x, approximate="tanh")}[kind]

    def timed(fn):
        for i in range(args.warmup):
            fn(sets[i % nsets])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(sets[i % nsets])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e6

    def torch_bwd(s):
        e = s["e"].detach().requires_grad_()
        g = s["g"].detach().requires_grad_()
        h = act(e) * g
        torch.autograd.grad(h, (e, g), s["dh"])

    res = {
        "fused_fwd_us": timed(lambda s: rope.glu_fwd(kind, s["e"], s["g"], out=s["h"])),
        "fused_bwd_us": timed(lambda s: rope.glu_bwd(kind, s["dh"], s["e"], s["g"], de=s["de"],
                                                     dg=s["dg"])),
        "torch_fwd_us": timed(lambda s: act(s["e"]) * s["g"]),
        "torch_fwd_bwd_us": timed(torch_bwd),
    }
    res["speedup_fwd"] = res["torch_fwd_us"] / res["fused_fwd_us"]
    res["speedup_fwd_bwd"] = res["torch_fwd_bwd_us"] / (res["fused_fwd_us"] + res["fused_bwd_us"])
    print(json.dumps({"compare": f"glu {kind} fused vs torch eager", "workload": w.name,
                      "dtype": w.dtype, **res}))


# The library's kGluPieceBlocks: a GLU call of 2x this many workgroups or more goes
# out as launches of about this many.
GLU_PIECE_BLOCKS = 32768


def glu_pieces(w) -> list:
    """Workgroups of each launch of one dense GLU call on workload w (1024 chunks of
    16 bytes, or of the row's widest dividing access, per workgroup; the library's
    glu_piece_blocks)."""
    vec = 16 // w.elem_bytes
    while (w.cols * w.elem_bytes) % (vec * w.elem_bytes):
        vec //= 2
    want = -(-(w.rows * (w.cols // vec)) // 1024)
    if want < 2 * GLU_PIECE_BLOCKS:
        return [want]
    n = -(-want // GLU_PIECE_BLOCKS)
    piece = (-(-want // n) + 7) // 8 * 8
    return [min(piece, want - b) for b in range(0, want, piece)]


def bench_glu(args) -> None:
    """One step = glu_fwd (e, g -> h) + glu_bwd (dh, e, g -> de, dg), out of place,
    on [tokens, intermediate] tensors resident in HBM; buffer sets rotate so no
    launch is served from the Infinity Cache. Prints one JSON line; the roofline is
    that of the backward (5 streams, the longer launch), the forward's is beside it."""
    import packed_varlen_rotary_rope_amd as rope

    w = workloads.glu_get(args.workload)
    dev = torch.device("cuda:0")
    n = w.elements
    set_bytes = 6 * n * w.elem_bytes
    nsets = max(2, math.ceil(8 * INFINITY_CACHE_BYTES / set_bytes))
    sets = []
    for i in range(nsets):
        st = {k: workloads.make_tensor((w.rows, w.cols), w.seed(k) + 100 * i, w.dtype, device=dev,
                                       chunk_rows=8192) for k in ("e", "g", "dh")}
        for k in ("h", "de", "dg"):
            st[k] = torch.empty((w.rows, w.cols), dtype=st["e"].dtype, device=dev)
        sets.append(st)
    stream = torch.cuda.current_stream(dev).cuda_stream
    kind = args.glu
    index_mode = {"auto": rope.INDEX_AUTO, "64": rope.INDEX_64}[args.index]

    def step(s, ev=None):
        if ev is not None:
            ev[0].record(stream)
        rope.glu_fwd(kind, s["e"], s["g"], out=s["h"], index_mode=index_mode)
        if ev is not None:
            ev[1].record(stream)
            ev[2].record(stream)
        rope.glu_bwd(kind, s["dh"], s["e"], s["g"], de=s["de"], dg=s["dg"], index_mode=index_mode)
        if ev is not None:
            ev[3].record(stream)

    if args.compare:
        return compare_glu_unfused(rope, w, kind, sets, nsets, args)
    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Per-launch durations after the timed region: forward-only and backward-only runs
    # of back-to-back launches, each between one pair of HIP events on the launch
    # stream (average, gaps included), then events around single launches of further
    # steps (minimum and median).
    reps = max(8, min(args.steps, 200))

    def region_us(launch):
        ev = [HipEvent(), HipEvent()]
        ev[0].record(stream)
        for i in range(reps):
            launch(sets[i % nsets])
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_ms(ev[1]) * 1e3 / reps

    fwd_us = region_us(lambda st: rope.glu_fwd(kind, st["e"], st["g"], out=st["h"],
                                              index_mode=index_mode))
    bwd_us = region_us(lambda st: rope.glu_bwd(kind, st["dh"], st["e"], st["g"], de=st["de"],
                                              dg=st["dg"], index_mode=index_mode))
    events = [[HipEvent() for _ in range(4)] for _ in range(min(args.steps, 100))]
    for i, ev in enumerate(events):
        step(sets[i % nsets], ev)
    torch.cuda.synchronize()
    fwd_all = [ev[0].elapsed_ms(ev[1]) * 1e3 for ev in events]
    bwd_all = [ev[2].elapsed_ms(ev[3]) * 1e3 for ev in events]
    fwd_bytes, bwd_bytes = 3 * n * w.elem_bytes, 5 * n * w.elem_bytes
    achieved = bwd_bytes / (bwd_us * 1e-6) / 1e9
    pieces = len(glu_pieces(w))  # launches per call
    out = {
        "metric": GLU_METRIC,
        "value": w.rows * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "arithmetic": f"{w.dtype} storage; activation and products in fp32",
        "data": "synthetic (seeded N(0,1) e, g, dh)",
        "config": {"workload": w.name, "rows": w.rows, "cols": w.cols, "kind": kind,
                   "buffer_sets": nsets, "index": args.index},
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": (read_traffic(GLU_TRAFFIC_FILE, GLU_SOURCES, "bwd_hbm_bytes_per_launch")
                        if kind == "swiglu" and w.name == "glu_qwen3_4b" else None),
            "kernel": "glu_kernel (backward)",
            "launches_per_call": pieces,
            "bytes_per_launch": bwd_bytes / pieces, "avg_launch_us": bwd_us / pieces,
            "avg_call_us": bwd_us,
            "timing": f"HIP events around {reps} back-to-back backward calls / ({reps} x "
                      "launches per call)",
            "min_call_us": float(np.min(bwd_all)), "median_call_us": float(np.median(bwd_all)),
        },
        "forward": {"launches_per_call": pieces, "bytes_per_launch": fwd_bytes / pieces,
                    "avg_launch_us": fwd_us / pieces, "avg_call_us": fwd_us,
                    "min_call_us": float(np.min(fwd_all)),
                    "median_call_us": float(np.median(fwd_all)),
                    "achieved_GBps": fwd_bytes / (fwd_us * 1e-6) / 1e9},
    }
    if args.cpu_seconds > 0:
        from oracle import glu as glu_oracle

        rows = max(1, min(w.rows, 256))
        host = {k: workloads.host_bits(workloads.make_tensor((rows, w.cols), w.seed(k), w.dtype))
                for k in ("e", "g", "dh")}
        nthreads = max(1, min(16, len(os.sched_getaffinity(0))))

        def one(threads):
            return lambda: glu_oracle.seconds(kind, host["e"], host["g"], host["dh"], w.dtype,
                                              threads)

        reps, total = _timed_reps(one(nthreads), args.cpu_seconds, 100000)
        reps1, total1 = _timed_reps(one(1), args.cpu_seconds / 4, 100000)
        out["cpu_baseline"] = {
            "value": rows * reps / total, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{reps} fwd+bwd passes over {rows} of the {w.rows} rows "
                      f"({w.cols} columns), {total:.1f} s timed",
            "value_1_core": rows * reps1 / total1, "cpu_model": cpu_model(),
        }
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None,
                    choices=workloads.names() + workloads.glu_names(),
                    help=f"default: {HEADLINE_WORKLOAD} (glu_qwen3_4b with --glu)")
    ap.add_argument("--sweep", action="store_true",
                    help="time the default launch over a range of token counts (one sequence, "
                         "32+8 heads) with a torch in-place reference, fit t = t0 + b T, then exit")
    ap.add_argument("--sweep-summary", default=None, metavar="RUN_DIR",
                    help="write profiles/rope_qk_size_sweep.txt from RUN_DIR (rocprofv3 kernel "
                         "trace of --sweep and its JSON line in RUN_DIR/sweep.json), then exit")
    ap.add_argument("--head-shapes", action="store_true",
                    help="time the default launch on every head shape of HEAD_SHAPES (one "
                         "sequence each) beside torch's in-place reference; one JSON line")
    ap.add_argument("--head-shapes-summary", default=None, metavar="JSON",
                    help="write profiles/rope_qk_head_shapes.txt from the JSON line of "
                         "--head-shapes in this file, then exit")
    ap.add_argument("--configs", default="all", choices=["all", "none"],
                    help="all: also time every other RoPE workload's default launches and put "
                         "them in the JSON line (per_config); none: the chosen workload only")
    ap.add_argument("--tokens-per-wave", type=int, default=0, help="0: library default")
    ap.add_argument("--padded", default="compact", choices=["compact", "seqused"],
                    help="padded workloads (seqused): compact launches over the rotated tokens "
                         "only (rope_qk_apply_padded, with cu_valid made once per batch and "
                         "the host count of rotated tokens), or the seqused launch of the "
                         "plain entry point")
    ap.add_argument("--positions", default="cu", choices=["cu", "ids", "shards4"],
                    help="position source: cu_seqlens; explicit per-token ids; or the batch "
                         "cut into 4 token shards, each launched with per-sequence offsets")
    ap.add_argument("--pos-scale", type=float, default=1.0,
                    help="linear position interpolation factor (>= 1)")
    ap.add_argument("--layout", default="contiguous", choices=["contiguous", "qkv"],
                    help="qkv: Q/K (and dQ/dK) are strided views into fused QKV buffers")
    ap.add_argument("--index", default="auto", choices=["auto", "64"],
                    help="64: force the 64-bit offset specialization (auto: 64-bit only when needed)")
    ap.add_argument("--cos-sin", default="fly", choices=["fly", "table"],
                    help="fly: cos/sin evaluated in the kernel (default); table: read from a "
                         "cos/sin cache made once with the library's export (rope_qk_apply_table)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph instead of launching it "
                         "eagerly from Python")
    ap.add_argument("--glu", default=None, choices=["swiglu", "geglu", "geglu_tanh"],
                    help="time the SwiGLU/GeGLU kernels instead (workload: a glu_* name)")
    ap.add_argument("--compare", action="store_true",
                    help="time the fused kernels against unfused variants, then exit")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="timed oracle work for cpu_baseline (0 disables it)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="only run a plain copy of this many GiB (PMC scale factor), then exit")
    ap.add_argument("--traffic-summary", nargs=4, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write the PMC traffic summary from rocprofv3 counter CSVs, then exit")
    ap.add_argument("--traffic-command", default="", help="commands recorded in that summary")
    ap.add_argument("--traffic-ea", nargs=4, default=None,
                    metavar=("EA_READ_CSV", "EA_WRITE_CSV", "COPY_EA_READ_CSV", "COPY_EA_WRITE_CSV"),
                    help="with --traffic-summary: also derive bytes from TCC-to-memory request "
                         "counts (the second counter family)")
    ap.add_argument("--traffic-kernel", default="rope", choices=["rope", "glu"],
                    help="which kernel's summary --traffic-summary writes")
    ap.add_argument("--trace-summary", default=None, metavar="KERNEL_TRACE_CSV",
                    help="write profiles/rope_qk_<workload>_kernel_trace.txt from a rocprofv3 "
                         "--kernel-trace CSV of a run on --workload, then exit")
    ap.add_argument("--trace-command", default="", help="command recorded in that summary")
    ap.add_argument("--glu-trace-summary", default=None, metavar="RUN_DIR",
                    help="write the GLU kernel-trace summary from RUN_DIR/glu_trace_<kind> and "
                         "RUN_DIR/glu_bench_<kind>.log, then exit")
    ap.add_argument("--glu-valu-summary", default=None, metavar="RUN_DIR",
                    help="write the GLU VALU-occupancy summary from RUN_DIR/<kind> PMC folders, "
                         "then exit")
    ap.add_argument("--padded-counters-summary", nargs=4, default=None,
                    metavar=("PADDED_DIR", "PACKED_DIR", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write the padded-vs-packed counter summary from rocprofv3 --pmc and "
                         "--kernel-trace output folders, then exit")
    ap.add_argument("--counters-summary", nargs=4, default=None,
                    metavar=("FLY_DIR", "TABLE_DIR", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write the cos/sin fly-vs-table counter summary from rocprofv3 "
                         "--pmc and --kernel-trace output folders, then exit")
    args = ap.parse_args()

    if args.sweep_summary:
        write_sweep_summary(args.sweep_summary, args.trace_command)
        return
    if args.head_shapes_summary:
        write_head_shapes_summary(args.head_shapes_summary, args.trace_command)
        return
    if args.glu_valu_summary:
        write_glu_valu_summary(args.glu_valu_summary, args.trace_command)
        return
    if args.glu_trace_summary:
        write_glu_trace_summary(args.glu_trace_summary, args.trace_command)
        return
    if args.padded_counters_summary:
        write_padded_counters_summary(*args.padded_counters_summary, command=args.trace_command)
        return
    if args.counters_summary:
        write_counters_summary(*args.counters_summary, command=args.trace_command)
        return

    if args.trace_summary:
        write_trace_summary(args.trace_summary, args.workload or "qwen3_4b_packed",
                            args.trace_command)
        return

    if args.traffic_summary:
        if args.traffic_kernel == "glu":
            write_glu_traffic_summary(*args.traffic_summary, command=args.traffic_command)
        else:
            write_traffic_summary(*args.traffic_summary, command=args.traffic_command,
                                  workload=args.workload or HEADLINE_WORKLOAD, ea=args.traffic_ea)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration, 5)
        return
    if args.glu:
        args.workload = args.workload or "glu_qwen3_4b"
        if args.workload not in workloads.glu_names():
            raise SystemExit("--glu takes a glu_* workload")
        return bench_glu(args)
    args.workload = args.workload or HEADLINE_WORKLOAD
    if args.workload not in workloads.names():
        raise SystemExit("glu_* workloads need --glu")

    import packed_varlen_rotary_rope_amd as rope

    dev = torch.device("cuda:0")
    if args.sweep:
        print(json.dumps(size_sweep(rope, dev, max(50, min(args.steps, 500)))))
        return
    if args.head_shapes:
        print(json.dumps(head_shape_survey(rope, dev, max(50, min(args.steps, 500)))))
        return
    w = workloads.get(args.workload)
    set_bytes = 2 * w.T * (w.Hq + w.Hkv) * w.D * w.elem_bytes  # Q, K, dQ, dK
    # Enough sets that a buffer is touched again only after >= 8x the Infinity
    # Cache's capacity of other traffic: no launch can be served from it.
    nsets = max(2, math.ceil(8 * INFINITY_CACHE_BYTES / set_bytes))
    cu, su, sets = make_sets(w, nsets, dev, args.layout)
    tpw = args.tokens_per_wave

    stream = torch.cuda.current_stream(dev).cuda_stream  # the stream the library launches on
    if args.compare:
        if args.layout != "contiguous":
            raise SystemExit("--compare measures contiguous Q/K only")
        return compare_unfused(rope, w, cu, su, sets, nsets, args, stream)

    pid = None
    shards = None
    if args.positions == "ids":
        pid = torch.from_numpy(packed_position_ids(w)).to(dev)
    elif args.positions == "shards4":
        if su is not None:
            raise SystemExit("--positions shards4 needs a fully packed workload (no seqused)")
        # 4 token ranges; a sequence crossing a cut continues in the next shard with
        # the global position of its first token there as offset.
        bounds = [w.T * r // 4 for r in range(5)]
        shards = []
        cu_np = w.cu_seqlens.astype(np.int64)
        for a, b in zip(bounds[:-1], bounds[1:]):
            starts = np.clip(cu_np[:-1], a, b)
            ends = np.clip(cu_np[1:], a, b)
            keep = ends > starts
            cu_r = np.concatenate([[0], np.cumsum((ends - starts)[keep])]).astype(np.int32)
            off_r = (starts - cu_np[:-1])[keep].astype(np.int32)
            shards.append((a, b, torch.from_numpy(cu_r).to(dev), torch.from_numpy(off_r).to(dev)))

    index_mode = {"auto": rope.INDEX_AUTO, "64": rope.INDEX_64}[args.index]

    tables = None
    if args.cos_sin == "table":
        if shards is not None or args.pos_scale != 1.0:
            raise SystemExit("--cos-sin table times the cu_seqlens / ids position sources, "
                             "unscaled")
        # The cos/sin cache a caller would keep: every position of the batch, made
        # once by the library's own export, outside the timed region.
        rows = int(max(w.lengths))
        tables = rope.cos_sin_table(rows, w.D, w.theta, dev)

    compact = compact_launch(w, args.padded) and tpw == 0 and pid is None and shards is None \
        and tables is None
    if compact:
        cv, valid = padded_metadata(rope, w, cu, su)
    # launches per pass: one per call, or the row-group kernel's pieces of a long pass
    if tpw != 0 or not group_geometry(w) or (su is not None and not compact and pid is None):
        pieces = len(shards) if shards is not None else 1
    elif shards is not None:
        pieces = sum(len(group_pieces(b - a, w)) for a, b, _, _ in shards)
    else:
        pieces = len(group_pieces(w.valid_tokens if compact else w.T, w))

    def launch(qt, kt, direction):
        if compact:
            rope.qk_apply_padded_(qt, kt, w.theta, direction, cu, su, cv, valid,
                                  pos_scale=args.pos_scale, index_mode=index_mode)
        elif tables is not None:
            rope.qk_apply_table_(qt, kt, tables[0], tables[1], direction,
                                 cu_seqlens=None if pid is not None else cu,
                                 seqused=None if pid is not None else su, position_ids=pid,
                                 tokens_per_wave=tpw, index_mode=index_mode)
        elif shards is not None:
            for a, b, cu_r, off_r in shards:
                rope.qk_apply_ex_(qt[a:b], kt[a:b], w.theta, direction, cu_seqlens=cu_r,
                                  seq_offsets=off_r, pos_scale=args.pos_scale,
                                  tokens_per_wave=tpw, index_mode=index_mode)
        elif pid is not None or args.pos_scale != 1.0 or args.layout == "qkv":
            rope.qk_apply_ex_(qt, kt, w.theta, direction, cu_seqlens=None if pid is not None else cu,
                              seqused=None if pid is not None else su, position_ids=pid,
                              pos_scale=args.pos_scale, tokens_per_wave=tpw,
                              index_mode=index_mode)
        else:
            rope.qk_apply_(qt, kt, cu, w.theta, direction, seqused=su, tokens_per_wave=tpw,
                           index_mode=index_mode)

    def step(s, ev=None):
        if ev is not None:
            ev[0].record(stream)
        launch(s["q"], s["k"], 1)
        if ev is not None:
            ev[1].record(stream)
            ev[2].record(stream)
        launch(s["dq"], s["dk"], -1)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()

    # The timed region: K steps back to back, bracketed by synchronize (wall clock)
    # and by one pair of HIP events on the launch stream (GPU time). Nothing else is
    # enqueued between the launches.
    run = step
    if args.graph:
        # One HIP graph per buffer set, each holding one step (forward + backward
        # launches), captured on torch's capture stream; replayed in the same rotation.
        graphs = []
        torch.cuda.synchronize()
        for st in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(st)
            graphs.append(g)
        torch.cuda.synchronize()
        by_set = {id(st): g for st, g in zip(sets, graphs)}

        def run(st):
            by_set[id(st)].replay()

        for i in range(max(args.warmup, nsets)):
            run(sets[i % nsets])
    region = [HipEvent(), HipEvent()]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(args.steps):
        run(sets[i % nsets])
    region[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region_s = region[0].elapsed_ms(region[1]) / 1e3
    # Average duration of one pass (forward or backward: one launch, or one per shard
    # with --positions shards4, or the row-group kernel's pieces of a long pass) and
    # of one launch, gaps between launches included.
    avg_pass_s = region_s / (2 * args.steps)
    avg_launch_s = avg_pass_s / pieces
    bpp = algorithmic_bytes_per_pass(w)
    bpl = bpp / pieces
    achieved = bpl / avg_launch_s / 1e9

    # Sampled per-pass durations, after the timed region: HIP events around both
    # passes of each of up to 250 further steps (context: minimum and median).
    events = [[HipEvent() for _ in range(4)] for _ in range(min(250, args.steps))]
    for i, ev in enumerate(events):
        step(sets[i % nsets], ev)
    torch.cuda.synchronize()
    launch_ms = []
    for ev in events:
        launch_ms.append(ev[0].elapsed_ms(ev[1]))
        launch_ms.append(ev[2].elapsed_ms(ev[3]))
    tokens_per_step = w.valid_tokens
    value = tokens_per_step * args.steps / elapsed
    ms_per_step = elapsed / args.steps * 1e3
    # the PMC traffic summary covers the default configuration of this workload only
    default_config = (args.positions == "cu" and args.pos_scale == 1.0 and tpw == 0
                      and args.layout == "contiguous" and args.index == "auto"
                      and args.cos_sin == "fly" and not args.graph)
    traffic = read_traffic(traffic_path(w.name)) if default_config else None
    # the torch in-place elementwise reference over the same bytes, same buffer sets
    ref_us = None
    if w.seqused is None and args.layout == "contiguous":
        ref_us = inplace_reference_us(sets, nsets, stream, 2 * max(args.steps, 20))

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "arithmetic": f"{w.dtype} storage; rotation in fp32 (FMA-compensated), cos/sin "
                      "correctly rounded to fp32 from fp64 arithmetic",
        "data": "synthetic (seeded N(0,1) Q/K/dQ/dK, seeded length draws)",
        "config": {
            "workload": w.name,
            "T": w.T, "valid_tokens": w.valid_tokens, "num_seqs": w.num_seqs,
            "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "theta": w.theta,
            "buffer_sets": nsets, "tokens_per_wave": tpw or "auto",
            "positions": args.positions, "pos_scale": args.pos_scale,
            "layout": args.layout, "index": args.index, "cos_sin": args.cos_sin,
            **({"padded_launch": "compact" if compact else "seqused"}
               if w.seqused is not None else {}),
            "launch": "hip graph per step" if args.graph else "eager",
        },
        "step_hbm_GBps": 2 * bpp * args.steps / elapsed / 1e9,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "kernel": rope_kernel_name(w, tpw, args.padded if compact else "seqused"),
            "launches_per_pass": pieces,
            "bytes_per_launch": bpl,
            "avg_launch_us": avg_launch_s * 1e6,
            "avg_pass_us": avg_pass_s * 1e6,
            "timing": "HIP events around the timed region / (2 x steps x launches per pass)",
            "sampled_passes": len(launch_ms),
            "sampled_avg_pass_us": float(np.mean(launch_ms)) * 1e3,
            "sampled_median_pass_us": float(np.median(launch_ms)) * 1e3,
            "sampled_min_pass_us": float(np.min(launch_ms)) * 1e3,
        },
    }
    if ref_us is not None:
        out["roofline"]["frac_of_ceiling"] = ref_us / (avg_pass_s * 1e6)
        out["roofline"]["ceiling_reference"] = {
            "op": "torch in-place neg_ on Q, then on K (same bytes as one pass)",
            "avg_pass_us": ref_us, "GBps": bpp / (ref_us * 1e-6) / 1e9,
            "frac_of_ceiling": "reference time / RoPE pass time"}
    if args.cpu_seconds > 0:
        nthreads = max(1, min(16, len(os.sched_getaffinity(0))))
        if w.T * (w.Hq + w.Hkv) * w.D > 2 ** 28:  # too large to process whole on the host
            out["cpu_baseline"] = cpu_baseline_sampled(w, sets[0], args.cpu_seconds, nthreads)
        else:
            out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, nthreads)
    if args.configs == "all" and default_config:
        del sets, events
        torch.cuda.empty_cache()
        per = {}
        for name in SUB_WORKLOADS:
            if name == w.name:
                per[name] = {
                    "T": w.T, "valid_tokens": w.valid_tokens, "Hq": w.Hq, "Hkv": w.Hkv,
                    "D": w.D, "dtype": w.dtype,
                    "kernel": rope_kernel_name(w, 0, args.padded if compact else "seqused"),
                    "index": "64-bit" if needs_long_index(w) else "32-bit",
                    "launches_per_pass": pieces, "bytes_per_launch": bpl,
                    "avg_launch_us": avg_launch_s * 1e6, "avg_pass_us": avg_pass_s * 1e6,
                    "GBps": achieved, "frac": achieved / HBM_PEAK_GBPS,
                    "fwd_bwd_tokens_per_s": w.valid_tokens / (2 * avg_pass_s),
                    "passes_timed": 2 * args.steps, "headline": True}
                if ref_us is not None:
                    per[name]["torch_inplace_us"] = ref_us
                    per[name]["frac_of_ceiling"] = ref_us / (avg_pass_s * 1e6)
                continue
            sw = workloads.get(name)
            print(f"[bench] timing {name}", file=sys.stderr, flush=True)
            per[name] = time_workload(rope, sw, dev, 200, 20, padded=args.padded)
        if "qwen3_8b_padded" in per and "qwen3_8b_packed" in per:
            pad, pk = per["qwen3_8b_padded"], per["qwen3_8b_packed"]
            pad["t_over_packed"] = pad["avg_pass_us"] / pk["avg_pass_us"]
            pad["valid_fraction"] = pad["valid_tokens"] / pad["T"]
        out["per_config"] = per
    print(json.dumps(out))


if __name__ == "__main__":
    main()
