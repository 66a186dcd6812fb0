"""rocprofv3 evidence for the fp4q kernels.

    python -m fp4_post_quantization_amd.evidence run --config c2 --out DIR
    python -m fp4_post_quantization_amd.evidence summarize --config c2 --in DIR --profiles profiles

``run`` profiles ``bench.py --config <config>`` four times, each in a pass of
its own: a kernel trace with statistics, one counter pass for the VALU
(SQ_WAVES, SQ_INSTS_VALU, SQ_ACTIVE_INST_VALU, SQ_BUSY_CYCLES,
GRBM_GUI_ACTIVE), one for FETCH_SIZE and one for WRITE_SIZE.  The bench
also runs a plain elementwise kernel that reads and writes 256 MiB once
(``--copy-calib``); its counter readings give the factors that turn
FETCH_SIZE / WRITE_SIZE into bytes.

``summarize`` writes ``<profiles>/<stem>.md`` (durations, VALU issue
utilisation, calibrated HBM traffic per dispatch) and ``<stem>.traffic.json``
(the dominant kernel's calibrated traffic, tagged with a hash of the kernel
sources so that it is only reported while the kernels are unchanged).

This module starts rocprofv3 as a child process and never touches the GPU
itself.
"""

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
KERNEL_SOURCES = [os.path.join(PKG, "csrc", "fp4q.hip"), os.path.join(PKG, "csrc", "fp4q_device.h"),
                  os.path.join(ROOT, "include", "fp4q.h")]
GEMM_SOURCES = [os.path.join(PKG, "csrc", "fp4q_gemm.hip"), os.path.join(ROOT, "include", "fp4q_gemm.h")]

VALU_COUNTERS = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
PASSES = {
    "trace": ["--kernel-trace", "--stats"],
    "valu": ["--pmc", *VALU_COUNTERS],
    "fetch": ["--pmc", "FETCH_SIZE"],
    "write": ["--pmc", "WRITE_SIZE"],
}
COPY_BYTES = 256 * 2**20  # bench.py --copy-calib: one read and one write of 256 MiB

# (N, K) of the projections of an 8B-shaped layer by GEMM kernel instantiation, and the widths of
# its four activation inputs
_W4A4_BIG = "mx_gemm_ring_kernel<2, 4, 4, 2, 2, unsigned short, true, 128, true, true>"
_W4A4_SMALL = "mx_gemm_ring_kernel<2, 2, 2, 2, 2, unsigned short, true, 128, false, false>"
_W4A4_NK_BIG = [(4096, 4096), (4096, 4096), (14336, 4096), (14336, 4096), (4096, 14336)]
_W4A4_NK_SMALL = [(1024, 4096), (1024, 4096)]
_W4A4_IN = [4096, 4096, 4096, 14336]


# NVFP4 W4A4 layer: q, o, gate, up, down through the decode pass and the bf16 ring (256 x 256 tiles)
_W4A4NV_BIG = "mx_gemm_ring_kernel<2, 4, 4, 2, 2, unsigned short, false, 128, false, true>"
# k, v: NVFP4 codes staged in LDS and decoded in registers (128 x 128 tiles)
_W4A4NV_SMALL = "nv_gemm_ring_kernel<2, 2, 2, 2, 4, unsigned short>"
# decode passes: per large product one of A (8192 x K) and one of B (N x K): codes + scales in,
# bf16 out
_W4A4NV_DECODE = [8192 * k for n, k in _W4A4_NK_BIG] + [n * k for n, k in _W4A4_NK_BIG]


def _bf16_gemm_mean(nks, what, m=8192):
    vals = [2 * m * n * k if what == "flops" else (m + n) * k * 2 + m * n * 2 for n, k in nks]
    return sum(vals) / len(vals)


def _nv_codes_gemm_mean(nks, what, m=8192):
    # NVFP4 operands read as codes + E4M3 scales (one byte per 16 elements), bf16 output
    vals = [2 * m * n * k if what == "flops" else (m + n) * k * (0.5 + 1 / 16) + m * n * 2 for n, k in nks]
    return sum(vals) / len(vals)


def _gemm_mean(nks, what, m=8192):
    vals = [2 * m * n * k if what == "flops" else m * k * (0.5 + 1 / 32) + n * k * (0.5 + 1 / 32) + m * n * 2
            for n, k in nks]
    return sum(vals) / len(vals)


def panel_fetch(m, n, row_bytes, bm, bn, resident=32, xcds=8, group_rows=8):
    """Bytes one ring-GEMM dispatch fetches into the XCDs' L2 caches if each L2 holds the operand
    panels (BM or BN rows x all of K) of the tiles its XCD runs at once, and nothing from one such
    round to the next (a round's panels exceed the 4 MB L2).  Workgroup i runs on XCD i % xcds;
    the kernel numbers an XCD's tiles contiguously, in groups of group_rows tile rows walked column
    by column (as the GEMM source's tile order does), and the XCD's `resident` workgroups (one per
    CU) hold consecutive numbers.  Each round then fetches its distinct A and B panels once."""
    tiles_m, tiles_n = -(-m // bm), -(-n // bn)
    per, rem = divmod(tiles_m * tiles_n, xcds)
    total = 0
    for x in range(xcds):
        start = x * (per + 1) if x < rem else rem * (per + 1) + (x - rem) * per
        count = per + (1 if x < rem else 0)
        for r0 in range(0, count, resident):
            rows, cols = set(), set()
            for lin in range(start + r0, start + min(count, r0 + resident)):
                group = lin // (group_rows * tiles_n)
                first = group * group_rows
                gsize = min(tiles_m - first, group_rows)
                r = lin - group * group_rows * tiles_n
                rows.add(first + r % gsize)
                cols.add(r // gsize)
            total += (sum(min(bm, m - t * bm) for t in rows) + sum(min(bn, n - t * bn) for t in cols)) * row_bytes
    return total


def _panel_mean(nks, bytes_per_k, tile, m=8192):
    vals = [panel_fetch(m, n, k * bytes_per_k, tile, tile) for n, k in nks]
    return sum(vals) / len(vals)

# dominant kernel and algorithmic bytes per dispatch of each workload
WORKLOADS = {
    "c2": {"stem": "nvfp4_wmse_bf16_4096x4096", "kernel": "nvfp4_sweep_kernel",
           "title": "NVFP4 WMSE ScaleSweep, bf16 4096x4096, offsets [-8,+7]",
           "alg_bytes": {"nvfp4_sweep_kernel": 4096 * 4096 * (2 + 0.5 + 6 / 16),
                         "amax_flat_kernel": 4096 * 4096 * 2}},
    "c3a": {"stem": "mxfp4_bf16_8192x4096", "kernel": "mxfp4_sweep_kernel",
            "title": "MXFP4 exponent window [-1,0], bf16 8192x4096 activations",
            "alg_bytes": {"mxfp4_sweep_kernel": 8192 * 4096 * (2 + 0.5 + 6 / 32)}},
    # GPTQ on 4096 x 4096 (1024-column blocks of eight 128-column batches).  Per dispatch, averaged
    # over a call: the 12 near updates of the block-internal binary tree (per block two of the next
    # 256 columns with the last two batches' errors, one of the next 512 with the last four's: read
    # and write W[:, N], read the K error columns and U[K rows, N]; fp32 MFMA), the 3 far updates
    # (all later columns, L = 3072, 2048, 1024, with the block's 1024 error columns and
    # U[block, later]; bf16 MFMA on operands split in three, six bf16 products per fp32 product) and
    # the 32 batch kernels (read and write 128 columns, write codes and scales, read U's 128 x 128
    # block; the odd batches of a block first apply the previous batch's errors to their columns,
    # reading those 128 error columns and another 128 x 128 block of U)
    "gptq": {"stem": "gptq_nvfp4_f32_4096x4096", "kernel": "gptq_update_split_kernel",
             "title": "GPTQ with ScaleSweep group scales, fp32 4096x4096, MSE and WMSE",
             "alg_bytes": {"gptq_update_kernel": sum(c * (4096 * n * 8 + 4096 * n * 4 + n * n * 4)
                                                     for c, n in ((8, 256), (4, 512))) / 12,
                           "gptq_update_split_kernel": sum(4096 * L * 8 + 4096 * 1024 * 4 + 1024 * L * 4
                                                           for L in (1024, 2048, 3072)) / 3,
                           "gptq_batch_kernel": 4096 * 128 * 8 + 4096 * 64 + 4096 * 8 + 128 * 128 * 4
                                                + (4096 * 128 * 4 + 128 * 128 * 4) / 2},
             "alg_flops": {"gptq_update_kernel": sum(c * 2 * 4096 * n * n for c, n in ((8, 256), (4, 512))) / 12,
                           "gptq_update_split_kernel": sum(6 * 2 * 4096 * 1024 * L for L in (1024, 2048, 3072)) / 3},
             "extra_counters": ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES"],
             "peak_tflops": {"gptq_update_kernel": 157.3, "gptq_update_split_kernel": 2500.0},
             "peak_label": "the published dense figure of the kernel's MFMA type: fp32 157.3 TFLOP/s for the "
                           "near update, bf16 2500 TFLOP/s for the far update, whose flops count its six bf16 "
                           "products per fp32 product"},
    # W4A4 8B layer at 8192 tokens.  Per GEMM dispatch: A (codes + scales) + B (codes + scales)
    # + C (bf16), flops 2 M N K, averaged over the projections each kernel instantiation serves
    # (256 x 256 tiles: q, o, gate, up, down; 128 x 128 tiles: k, v).  The activation quantizer
    # reads bf16 and writes codes, scales and offsets (mean over the four inputs).
    "w4a4": {"stem": "mxfp4_w4a4_gemm_8b_layer_8192tok", "kernel": _W4A4_BIG,
             "title": "W4A4 MXFP4 layer (8B shapes, 8192 tokens): scaled-FP4 MFMA GEMMs + activation quantization",
             "alg_bytes": {_W4A4_BIG: _gemm_mean(_W4A4_NK_BIG, "bytes"), _W4A4_SMALL: _gemm_mean(_W4A4_NK_SMALL, "bytes"),
                           "mxfp4_sweep_kernel": sum(8192 * k * (2 + 0.5 + 2 / 32) for k in _W4A4_IN)
                           / len(_W4A4_IN)},
             "alg_flops": {_W4A4_BIG: _gemm_mean(_W4A4_NK_BIG, "flops"),
                           _W4A4_SMALL: _gemm_mean(_W4A4_NK_SMALL, "flops")},
             "extra_counters": ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES"],
             "peak_tflops": 10100.0, "peak_label": "the published dense FP4 (MXFP4 scaled MFMA) figure",
             "panel_fetch": {_W4A4_BIG: _panel_mean(_W4A4_NK_BIG, 0.5 + 1 / 32, 256)},
             "sources": GEMM_SOURCES},
    "w4a4nv": {"stem": "nvfp4_w4a4_gemm_8b_layer_8192tok", "kernel": _W4A4NV_BIG,
               "title": "W4A4 NVFP4 layer (8B shapes, 8192 tokens): bf16-decoded operands on the bf16 matrix cores",
               "alg_bytes": {_W4A4NV_BIG: _bf16_gemm_mean(_W4A4_NK_BIG, "bytes"),
                             _W4A4NV_SMALL: _nv_codes_gemm_mean(_W4A4_NK_SMALL, "bytes"),
                             "nvfp4_to_bf16_kernel": sum(e * (0.5 + 1 / 16 + 2) for e in _W4A4NV_DECODE)
                             / len(_W4A4NV_DECODE)},
               "alg_flops": {_W4A4NV_BIG: _bf16_gemm_mean(_W4A4_NK_BIG, "flops"),
                             _W4A4NV_SMALL: _nv_codes_gemm_mean(_W4A4_NK_SMALL, "flops")},
               "extra_counters": ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES"],
               "peak_tflops": 2500.0, "peak_label": "the published dense bf16/fp16 figure (the operands run on "
                                                    "the bf16 and fp16 matrix cores)",
               "panel_fetch": {_W4A4NV_BIG: _panel_mean(_W4A4_NK_BIG, 2, 256)},
               "sources": GEMM_SOURCES},
    # FOCUS forward quantizer on the c2 weight: x (bf16), FP16 coefficients per 8, E4M3 scales in;
    # codes and the float32 dequantized output out
    "focus": {"stem": "focus_relaxed_bf16_4096x4096", "kernel": "relaxed_quant_kernel",
              "title": "FOCUS forward quantizer, NVFP4, bf16 4096x4096, sub-blocks of 8, dequantized output",
              "alg_bytes": {"relaxed_quant_kernel": 4096 * 4096 * (2 + 2 / 8 + 1 / 16 + 0.5 + 4)}},
    # one 70B-shaped gate projection with a fused 16-point Hadamard and the WMSE sweep
    "c5gate": {"stem": "nvfp4_wmse_h16_bf16_28672x8192", "kernel": "nvfp4_sweep_kernel",
               "title": "NVFP4 WMSE ScaleSweep after a 16-point block Hadamard, bf16 28672x8192 (70B gate)",
               "alg_bytes": {"nvfp4_sweep_kernel": 28672 * 8192 * (2 + 0.5 + 6 / 16),
                             "amax_chunks_kernel": 28672 * 8192 * 2}},
    "c3b": {"stem": "mxfp4_absmax_bf16_8192x4096", "kernel": "mxfp4_sweep_kernel",
            "title": "MXFP4 AbsMax window [0,0], bf16 8192x4096 activations",
            "alg_bytes": {"mxfp4_sweep_kernel": 8192 * 4096 * (2 + 0.5 + 6 / 32)}},
}


def _code_only(text):
    """C/C++ source with comments and whitespace removed (string literals in
    these sources contain no comment markers)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def source_hash(config=None):
    """sha256 over the code (comments and whitespace removed) of the sources
    of the workload's dominant kernel."""
    h = hashlib.sha256()
    for p in WORKLOADS.get(config, {}).get("sources", KERNEL_SOURCES):
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def bench_cmd(config, steps):
    # every call on one stream, so each kernel's traced duration is its own (the bench line's pipelined
    # steps overlap kernels of consecutive steps)
    return [sys.executable, os.path.join(ROOT, "bench.py"), "--config", config, "--steps", str(steps),
            "--warmup", "1", "--no-cpu-baseline", "--copy-calib", "--streams", "1"]


def passes(config):
    w = WORKLOADS.get(config, {})
    p = dict(PASSES)
    p["valu"] = ["--pmc", *VALU_COUNTERS, *w.get("extra_counters", [])]
    return p


def rocprof_cmd(name, out_dir, config, steps):
    return ["rocprofv3", *passes(config)[name], "-d", os.path.join(out_dir, name), "-o", config,
            "--output-format", "csv", "--", *bench_cmd(config, steps)]


def run(config, out_dir, steps):
    os.makedirs(out_dir, exist_ok=True)
    env = dict(os.environ, TMPDIR=os.environ.get("TMPDIR", "/tmp"))
    for name in passes(config):
        cmd = rocprof_cmd(name, out_dir, config, steps)
        print("==", " ".join(cmd), flush=True)
        # each pass is bounded; a counter request the hardware cannot serve hangs
        subprocess.run(["timeout", "-s", "KILL", "240", *cmd], check=True, env=env)


def _ours(name):
    return "fp4q::" in name or "fp4q_gemm::" in name


def _short(name):
    base = name.split("(")[0].replace("void ", "")
    for ns in ("fp4q::", "fp4q_gemm::"):
        if base.startswith(ns):
            base = base[len(ns):]
    return base


def _counter_means(path):
    rows = list(csv.DictReader(open(path)))
    agg = collections.defaultdict(list)
    for r in rows:
        key = (r["Kernel_Name"], r["Grid_Size"], r["Counter_Name"])
        agg[key].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in agg.items()}


def _agent(path):
    for r in csv.DictReader(open(path)):
        if r.get("Agent_Type", "").upper().endswith("GPU") or r.get("Name", "").startswith("gfx"):
            return r
    return {}


def summarize(config, in_dir, profiles):
    w = WORKLOADS[config]
    trace_dir = os.path.join(in_dir, "trace")
    stats = list(csv.DictReader(open(os.path.join(trace_dir, f"{config}_kernel_stats.csv"))))
    agent = _agent(os.path.join(trace_dir, f"{config}_agent_info.csv"))
    simds = int(agent.get("Simd_Count", 1024))
    clk_mhz = float(agent.get("Max_Engine_Clk_Fcompute", 2400))
    xcc = int(agent.get("Num_Xcc", 8))
    cus = int(agent.get("Cu_Count", 256))
    # shader engines: SQ_BUSY_CYCLES is summed over them (4 per XCD on gfx950)
    ses = int(agent.get("Num_Shader_Engines", 0) or agent.get("Shader_Engines", 0) or 4 * xcc)
    valu = _counter_means(os.path.join(in_dir, "valu", f"{config}_counter_collection.csv"))
    fetch = _counter_means(os.path.join(in_dir, "fetch", f"{config}_counter_collection.csv"))
    write = _counter_means(os.path.join(in_dir, "write", f"{config}_counter_collection.csv"))

    def pick(table, kname, counter):
        # dispatch-weighted mean over every grid size of the kernel, matching
        # the trace's average duration (GPTQ's update grid shrinks per batch)
        tot, cnt = 0.0, 0
        for (k, grid, c), (v, n) in table.items():
            if c == counter and kname in k:
                tot += v * n
                cnt += n
        return (tot / cnt, cnt) if cnt else None

    # copy calibration: the int32 bitwise-NOT kernel of bench.py --copy-calib (runs recorded
    # before it existed used a float32 negation: the neg dispatch size seen most often)
    def pick_calib(table, counter):
        best = None
        for (k, grid, c), (v, n) in table.items():
            if c == counter and "bitwise_not" in k:
                return (v, n)
            if c == counter and "neg_kernel" in k and (best is None or n > best[1]):
                best = (v, n)
        return best

    cf = pick_calib(fetch, "FETCH_SIZE")
    cw = pick_calib(write, "WRITE_SIZE")
    f_factor = COPY_BYTES / (cf[0] * 1024) if cf else None
    w_factor = COPY_BYTES / (cw[0] * 1024) if cw else None

    lines = [f"# {w['title']}", "",
             f"Device: {agent.get('Name', '?')}, {cus} CUs, {simds} SIMDs, {xcc} XCDs, "
             f"max engine clock {clk_mhz:.0f} MHz.", "", "Commands (each a pass of its own):", ""]
    for name in passes(config):
        cmd = rocprof_cmd(name, in_dir, config, 20)
        cmd = ["python" if c == sys.executable else ("bench.py" if c.endswith("bench.py") else c) for c in cmd]
        lines.append("    " + " ".join(cmd))
    lines += ["", "run together by", "",
              f"    python -m fp4_post_quantization_amd.evidence run --config {config} --out {in_dir} --steps 20",
              "", "and summarized by", "",
              f"    python -m fp4_post_quantization_amd.evidence summarize --config {config} --in {in_dir}"
              f" --profiles profiles", "",
              "## Kernel durations (kernel trace)", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    durations = {}
    for r in stats:
        name = r["Name"]
        if not _ours(name) and "neg_kernel" not in name and "bitwise_not" not in name:
            continue
        avg = float(r["AverageNs"]) / 1000
        durations[name] = avg
        lines.append(f"| `{_short(name)}` | {r['Calls']} | {avg:.2f} | {float(r['MinNs'])/1000:.2f} "
                     f"| {float(r['MaxNs'])/1000:.2f} |")
    lines += ["", "## Counters per dispatch (averages)", "",
              "VALU issue = SQ_INSTS_VALU x 4 cycles (one wave64 VALU instruction per SIMD per 4 cycles) "
              "/ (SIMDs x trace duration x clock).  VALUBusy = the same instruction cycles / (SIMDs x "
              "SQ_BUSY_CYCLES / shader engines), i.e. within the cycles the shader engines held waves, "
              "both from the counter run; neither can exceed 100%.  (SQ_ACTIVE_INST_VALU is not used: it "
              "counts every wave with a VALU instruction in flight, so its ratio to SIMD cycles can pass "
              "100%.)", "",
              "| kernel | waves | VALU insts | VALU issue | VALUBusy | FETCH KiB | WRITE KiB | HBM bytes "
              "(calibrated) | algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|---|---|---|"]
    record = None
    fetched = {}  # calibrated FETCH_SIZE bytes per dispatch, by kernel
    for name, avg_us in durations.items():
        if not _ours(name):
            continue
        key = _short(name) if _short(name) in w["alg_bytes"] else _short(name).split("<")[0]
        insts = pick(valu, name, "SQ_INSTS_VALU")
        waves = pick(valu, name, "SQ_WAVES")
        sq_busy = pick(valu, name, "SQ_BUSY_CYCLES")
        fk = pick(fetch, name, "FETCH_SIZE")
        wk = pick(write, name, "WRITE_SIZE")
        issue = insts[0] * 4 / (simds * avg_us * 1e-6 * clk_mhz * 1e6) if insts else None
        busy = 100 * insts[0] * 4 / (simds * sq_busy[0] / ses) if (insts and sq_busy and sq_busy[0]) else None
        hbm = (fk[0] * 1024 * f_factor + wk[0] * 1024 * w_factor) if (fk and wk and f_factor) else None
        if fk and f_factor:
            fetched[name] = fk[0] * 1024 * f_factor
        alg = w["alg_bytes"].get(key)
        lines.append(
            f"| `{_short(name)}` | {waves[0]:.0f} | {insts[0]:.4g} | "
            f"{'' if issue is None else f'{100 * issue:.1f}%'} | {'' if busy is None else f'{busy:.1f}%'} | "
            f"{fk[0] if fk else float('nan'):.1f} | {wk[0] if wk else float('nan'):.1f} | "
            f"{'' if hbm is None else f'{hbm / 1e6:.2f} MB'} | {'' if alg is None else f'{alg / 1e6:.2f} MB'} | "
            f"{'' if (hbm is None or alg is None) else f'{hbm / alg:.3f}'} |")
        if w["kernel"] in name and hbm is not None:
            record = {"workload": config, "kernel": _short(name), "avg_us": avg_us, "fetch_kib": fk[0],
                      "write_kib": wk[0], "fetch_factor": f_factor, "write_factor": w_factor,
                      "traffic_bytes": hbm, "alg_bytes": alg, "valu_issue": issue, "valu_busy_pct": busy,
                      "source_sha256": source_hash(config)}
    if w.get("panel_fetch"):
        lines += ["", "## L2 panel model", "",
                  "Predicted = the bytes the XCDs' L2 caches fetch if each holds the A and B panels (tile rows "
                  "x all of K) of the 32 tiles its CUs run at once and nothing from one such round to the "
                  "next, with the kernel's XCD-contiguous tile order (`panel_fetch` in this module); "
                  "measured = calibrated FETCH_SIZE.  Agreement says the fetch above the algorithmic bytes "
                  "is the panels each round re-reads, which a 4 MB L2 per XCD cannot keep across rounds "
                  "(and which the 256 MB Infinity Cache may serve without HBM).", "",
                  "| kernel | predicted fetch | measured fetch | measured / predicted |", "|---|---|---|---|"]
        for name in durations:
            pf = w["panel_fetch"].get(_short(name))
            if pf is None:
                continue
            got = fetched.get(name)
            lines.append(f"| `{_short(name)}` | {pf / 1e6:.2f} MB | "
                         f"{'' if got is None else f'{got / 1e6:.2f} MB'} | "
                         f"{'' if got is None else f'{got / pf:.3f}'} |")
            if record is not None and w["kernel"] in name:
                record.update(panel_fetch_bytes=pf)
    if w.get("alg_flops"):
        one_peak = not isinstance(w["peak_tflops"], dict)
        peak_note = f" ({w['peak_tflops']:.0f} TFLOP/s at 2.4 GHz)" if one_peak else ""
        lines += ["", "## Matrix cores", "",
                  f"Achieved = mean algorithmic flops per dispatch / average duration; peak = "
                  f"{w.get('peak_label', 'the published dense figure')}{peak_note}.  MFMA busy share = "
                  "SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE / XCDs); cycles per MFMA = "
                  "SQ_VALU_MFMA_BUSY_CYCLES / SQ_INSTS_MFMA.", "",
                  "| kernel | flops per dispatch | achieved TFLOP/s | of peak | MFMA insts | cycles per MFMA | "
                  "MFMA busy share | GPU clock (GRBM) |", "|---|---|---|---|---|---|---|---|"]
        for name, avg_us in durations.items():
            base = _short(name).split("<")[0]
            fl = w["alg_flops"].get(_short(name), w["alg_flops"].get(base))
            if fl is None:
                continue
            peak = w["peak_tflops"].get(base) if isinstance(w["peak_tflops"], dict) else w["peak_tflops"]
            mi = pick(valu, name, "SQ_INSTS_MFMA")
            mb = pick(valu, name, "SQ_VALU_MFMA_BUSY_CYCLES")
            grbm = pick(valu, name, "GRBM_GUI_ACTIVE")
            tf = fl / (avg_us * 1e-6) / 1e12
            share = mb[0] / (simds * grbm[0] / xcc) if (mb and grbm) else None
            cpm = mb[0] / mi[0] if (mb and mi and mi[0]) else None
            lines.append(f"| `{_short(name)}` | {fl:.4g} | {tf:.0f} | {100 * tf / peak:.1f}% | "
                         f"{'' if mi is None else f'{mi[0]:.4g}'} | {'' if cpm is None else f'{cpm:.1f}'} | "
                         f"{'' if share is None else f'{100 * share:.1f}%'} | counter-run cycles "
                         f"{'' if grbm is None else f'{grbm[0] / xcc:.4g}'} per XCD |")
            if record is not None and w["kernel"] in name:
                record.update(alg_flops=fl, achieved_tflops=tf, peak_tflops=w["peak_tflops"])
    lines += ["", "## Copy calibration", "",
              f"Plain elementwise kernel reading and writing {COPY_BYTES // 2**20} MiB once: FETCH_SIZE "
              f"{cf[0] if cf else float('nan'):.1f} KiB (factor {f_factor if f_factor else float('nan'):.4f}), "
              f"WRITE_SIZE {cw[0] if cw else float('nan'):.1f} KiB (factor "
              f"{w_factor if w_factor else float('nan'):.4f}).", ""]
    os.makedirs(profiles, exist_ok=True)
    md = os.path.join(profiles, w["stem"] + ".md")
    with open(md, "w") as f:
        f.write("\n".join(lines))
    if record:
        with open(os.path.join(profiles, w["stem"] + ".traffic.json"), "w") as f:
            json.dump(record, f, indent=1)
    print(md)


def committed_traffic(config):
    """The calibrated traffic record for a workload if it was measured on the
    current kernel sources, else None."""
    w = WORKLOADS.get(config)
    if not w:
        return None
    path = os.path.join(ROOT, "profiles", w["stem"] + ".traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    return rec if rec.get("source_sha256") == source_hash(config) else None


# issue-rate passes over the headline workload (each within the 8-SQ-counter limit of one pass)
ISSUE_PASSES = {
    "p1": ["SQ_INSTS_VALU", "SQ_INSTS_VALU_CVT", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VALU2", "SQ_INSTS_LDS",
           "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES"],
    "p2": ["SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_SALU",
           "SQ_ACTIVE_INST_MISC", "SQ_INSTS_VALU_TRANS_F32", "SQ_IFETCH"],
}
ISSUE_KERNEL = "nvfp4_sweep_kernel<unsigned short, true, 0>"


def issue_cmd(name, out_dir):
    return ["rocprofv3", "--pmc", *ISSUE_PASSES[name], "-d", os.path.join(out_dir, name), "-o", name,
            "--output-format", "csv", "--", sys.executable, os.path.join(ROOT, "bench.py"), "--config", "c2",
            "--steps", "5", "--warmup", "1", "--no-cpu-baseline", "--streams", "1"]


def issue_run(out_dir):
    os.makedirs(out_dir, exist_ok=True)
    env = dict(os.environ, TMPDIR=os.environ.get("TMPDIR", "/tmp"))
    for name in ISSUE_PASSES:
        cmd = issue_cmd(name, out_dir)
        print("==", " ".join(cmd), flush=True)
        subprocess.run(["timeout", "-s", "KILL", "240", *cmd], check=True, env=env)


def issue_summarize(in_dir, profiles):
    """Issue-rate summary of the headline sweep kernel from the two passes:
    per-dispatch counter means, the shader engines' busy window, the VALU
    issue rate inside it and the instructions per block-candidate."""
    vals, counts = {}, {}
    agent = {}
    for name in ISSUE_PASSES:
        path = os.path.join(in_dir, name, f"{name}_counter_collection.csv")
        for (k, grid, c), (v, n) in _counter_means(path).items():
            if ISSUE_KERNEL.split("<")[0] in k and "unsigned short, true, 0>" in k:
                tot, cnt = vals.get(c, (0.0, 0))
                vals[c] = (tot + v * n, cnt + n)
                counts[name] = counts.get(name, 0) + n
        agent = agent or _agent(os.path.join(in_dir, name, f"{name}_agent_info.csv"))
    m = {c: t / n for c, (t, n) in vals.items()}
    simds = int(agent.get("Simd_Count", 1024))
    xcc = int(agent.get("Num_Xcc", 8))
    ses = int(agent.get("Num_Shader_Engines", 0) or agent.get("Shader_Engines", 0) or 4 * xcc)
    clk = float(agent.get("Max_Engine_Clk_Fcompute", 2400)) * 1e6
    busy = m["SQ_BUSY_CYCLES"] / ses
    issue = (m["SQ_INSTS_VALU"] / simds) / (busy / 4)
    waves = 16384
    lines = [f"# Issue-rate counters: `{ISSUE_KERNEL}`, NVFP4 WMSE, bf16 4096x4096", "",
             f"Device: {agent.get('Name', 'gfx950')}, {simds} SIMDs, {ses} shader engines ({xcc} XCDs), "
             f"max engine clock {clk / 1e6:.0f} MHz.", "",
             "Two counter passes over the headline workload with every call on one stream (each pass its own "
             f"run; averages over every dispatch of the kernel in the run: {counts.get('p1', 0)} and "
             f"{counts.get('p2', 0)} dispatches):", ""]
    for name in ISSUE_PASSES:
        cmd = issue_cmd(name, in_dir)
        lines.append("    " + " ".join("python" if c == sys.executable else ("bench.py" if c.endswith("bench.py") else c)
                                       for c in cmd))
    lines += ["", "run by", "", f"    python -m fp4_post_quantization_amd.evidence issue --out {in_dir}", "",
              "and summarized by", "",
              f"    python -m fp4_post_quantization_amd.evidence issue-summary --in {in_dir} --profiles profiles", "",
              "| counter (per dispatch) | value |", "|---|---|"]
    unit = {"SQ_WAIT_INST_LDS": " quad-cycles", "SQ_WAVE_CYCLES": " quad-cycles", "SQ_ACTIVE_INST_VALU": " quad-cycles",
            "SQ_ACTIVE_INST_VALU2": " quad-cycles", "SQ_ACTIVE_INST_SCA": " quad-cycles",
            "SQ_WAIT_INST_ANY": " quad-cycles", "SQ_BUSY_CYCLES": f" (sum over {ses} SEs)"}
    for c in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_SALU", "SQ_INSTS_LDS",
              "SQ_WAIT_INST_LDS", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VALU2",
              "SQ_ACTIVE_INST_SCA", "SQ_WAIT_INST_ANY"):
        if c in m:
            extra = f" ({100 * m[c] / m['SQ_INSTS_VALU']:.1f}% of VALU)" if c == "SQ_INSTS_VALU_CVT" else ""
            lines.append(f"| {c} | {m[c]:.4g}{unit.get(c, '')}{extra} |")
    lines += ["", "Derived:",
              f"- Busy window per SE: {m['SQ_BUSY_CYCLES']:.4g} / {ses} = {busy / 1e3:.1f} k cycles = "
              f"{busy / clk * 1e6:.1f} us at {clk / 1e9:.1f} GHz (the rest of the kernel's traced duration is "
              "launch ramp and drain).",
              f"- VALU issue inside the busy window: ({m['SQ_INSTS_VALU']:.4g} / {simds} SIMDs) / "
              f"({busy / 1e3:.1f} k / 4 quad-cycles) = **{100 * issue:.1f}%** of a SIMD's VALU issue slots "
              "(one wave64 VALU instruction per quad-cycle).",
              f"- Per lane and candidate (a lane owns one 16-element block; {waves} waves x 16 candidates): "
              f"{m['SQ_INSTS_VALU_CVT'] / (waves * 16):.1f} converts of "
              f"{m['SQ_INSTS_VALU'] / (waves * 16):.1f} VALU instructions (the candidate loop's 16 converts and "
              "60 other VALU, plus prologue and emit).",
              f"- LDS waits: {m['SQ_WAIT_INST_LDS']:.3g} quad-cycles, "
              f"{100 * m['SQ_WAIT_INST_LDS'] / m['SQ_WAVE_CYCLES']:.2f}% of wave-cycles."]
    md = "\n".join(lines) + "\n"
    with open(os.path.join(profiles, "nvfp4_wmse_bf16_4096x4096_issue.md"), "w") as f:
        f.write(md)
    print(md)


def overlap(trace_csv, gap_us=200.0):
    """Concurrency of this library's kernels in a rocprofv3 kernel trace
    (kernel_trace.csv): the dispatches are cut into bursts at idle gaps
    longer than gap_us, and for the three largest bursts the summed kernel
    durations are compared with the burst's wall time (above 1: kernels of
    different queues ran at the same time).  Returns one dict per burst."""
    rows = list(csv.DictReader(open(trace_csv)))
    ks = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"], r["Queue_Id"])
                for r in rows if _ours(r["Kernel_Name"]))
    bursts, cur, end = [], [], None
    for k in ks:
        if cur and k[0] - end > gap_us * 1e3:
            bursts.append(cur)
            cur = []
        cur.append(k)
        end = k[1] if end is None or not cur[:-1] else max(end, k[1])
    if cur:
        bursts.append(cur)
    out = []
    for b in sorted(bursts, key=len)[-3:]:
        wall = (max(e for _, e, _, _ in b) - min(s_ for s_, _, _, _ in b)) / 1e3
        busy = sum(e - s_ for s_, e, _, _ in b) / 1e3
        sweeps = sum(1 for k in b if "sweep_kernel" in k[2])
        out.append({"kernels": len(b), "sweeps": sweeps, "queues": sorted({k[3] for k in b}),
                    "wall_us": round(wall, 1), "kernel_us": round(busy, 1),
                    "concurrency": round(busy / wall, 3), "wall_us_per_sweep": round(wall / max(sweeps, 1), 2)})
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--config", default="c2")
    r.add_argument("--out", required=True)
    r.add_argument("--steps", type=int, default=20)
    s = sub.add_parser("summarize")
    s.add_argument("--config", default="c2")
    s.add_argument("--in", dest="in_dir", required=True)
    s.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    o = sub.add_parser("overlap")
    o.add_argument("--trace", required=True, help="a rocprofv3 kernel_trace.csv")
    i = sub.add_parser("issue")
    i.add_argument("--out", required=True)
    i2 = sub.add_parser("issue-summary")
    i2.add_argument("--in", dest="in_dir", required=True)
    i2.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()
    if a.cmd == "run":
        run(a.config, a.out, a.steps)
    elif a.cmd == "issue":
        issue_run(a.out)
    elif a.cmd == "issue-summary":
        issue_summarize(a.in_dir, a.profiles)
    elif a.cmd == "overlap":
        for b in overlap(a.trace):
            print(json.dumps(b))
    else:
        summarize(a.config, a.in_dir, a.profiles)


if __name__ == "__main__":
    main()
