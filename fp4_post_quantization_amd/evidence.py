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
_W4A4_BIG = "mx_gemm_ring_kernel<2, 4, 4, 2, 2, unsigned short, true, 128, true>"
_W4A4_SMALL = "mx_gemm_ring_kernel<2, 2, 2, 2, 3, unsigned short, true, 128, false>"
_W4A4_NK_BIG = [(4096, 4096), (4096, 4096), (14336, 4096), (14336, 4096), (4096, 14336)]
_W4A4_NK_SMALL = [(1024, 4096), (1024, 4096)]
_W4A4_IN = [4096, 4096, 4096, 14336]


# NVFP4 W4A4 layer: bf16 ring instantiations (256 x 256 tiles: q, o, gate, up, down; 128 x 128: k, v)
_W4A4NV_BIG = "mx_gemm_ring_kernel<2, 4, 4, 2, 2, unsigned short, false, 128, false>"
_W4A4NV_SMALL = "mx_gemm_ring_kernel<2, 2, 2, 2, 4, unsigned short, false, 64, false>"
# decode passes: per product one of A (8192 x K) and one of B (N x K): codes + scales in, bf16 out
_W4A4NV_DECODE = [8192 * k for n, k in _W4A4_NK_BIG + _W4A4_NK_SMALL] + [n * k for n, k in
                                                                         _W4A4_NK_BIG + _W4A4_NK_SMALL]


def _bf16_gemm_mean(nks, what, m=8192):
    vals = [2 * m * n * k if what == "flops" else (m + n) * k * 2 + m * n * 2 for n, k in nks]
    return sum(vals) / len(vals)


def _gemm_mean(nks, what, m=8192):
    vals = [2 * m * n * k if what == "flops" else m * k * (0.5 + 1 / 32) + n * k * (0.5 + 1 / 32) + m * n * 2
            for n, k in nks]
    return sum(vals) / len(vals)

# dominant kernel and algorithmic bytes per dispatch of each workload
WORKLOADS = {
    "c2": {"stem": "nvfp4_wmse_bf16_4096x4096", "kernel": "nvfp4_sweep_kernel",
           "title": "NVFP4 WMSE ScaleSweep, bf16 4096x4096, offsets [-8,+7]",
           "alg_bytes": {"nvfp4_sweep_kernel": 4096 * 4096 * (2 + 0.5 + 6 / 16),
                         "amax_flat_kernel": 4096 * 4096 * 2}},
    "c3b": {"stem": "mxfp4_bf16_8192x4096", "kernel": "mxfp4_sweep_kernel",
            "title": "MXFP4 exponent window [-1,0], bf16 8192x4096 activations",
            "alg_bytes": {"mxfp4_sweep_kernel": 8192 * 4096 * (2 + 0.5 + 6 / 32)}},
    # GPTQ: per-dispatch bytes averaged over the 31 updates of a call (1024-column blocks of eight
    # 128-column batches): 28 in-block updates (the rest of the block, r = 896 ... 128 columns: read
    # and write W[:, rest], read the batch's errors and U[batch, rest]) and 3 block updates (all later
    # columns, L = 3072, 2048, 1024, with the block's 1024 error columns and U[block, later]); and the
    # 32 batch kernels (read and write 128 columns, write codes and scales, read U's 128 x 128 block)
    "gptq": {"stem": "gptq_nvfp4_f32_4096x4096", "kernel": "gptq_update_kernel",
             "title": "GPTQ with ScaleSweep group scales, fp32 4096x4096, MSE and WMSE",
             "alg_bytes": {"gptq_update_kernel": (sum(4 * (4096 * r * 8 + 4096 * 128 * 4 + 128 * r * 4)
                                                      for r in range(128, 1024, 128))
                                                  + sum(4096 * L * 8 + 4096 * 1024 * 4 + 1024 * L * 4
                                                        for L in (1024, 2048, 3072))) / 31,
                           "gptq_batch_kernel": 4096 * 128 * 8 + 4096 * 64 + 4096 * 8 + 128 * 128 * 4}},
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
             "peak_tflops": 10100.0, "sources": GEMM_SOURCES},
    "w4a4nv": {"stem": "nvfp4_w4a4_gemm_8b_layer_8192tok", "kernel": _W4A4NV_BIG,
               "title": "W4A4 NVFP4 layer (8B shapes, 8192 tokens): bf16-decoded operands on the bf16 matrix cores",
               "alg_bytes": {_W4A4NV_BIG: _bf16_gemm_mean(_W4A4_NK_BIG, "bytes"),
                             _W4A4NV_SMALL: _bf16_gemm_mean(_W4A4_NK_SMALL, "bytes"),
                             "nvfp4_to_bf16_kernel": sum(e * (0.5 + 1 / 16 + 2) for e in _W4A4NV_DECODE)
                             / len(_W4A4NV_DECODE)},
               "alg_flops": {_W4A4NV_BIG: _bf16_gemm_mean(_W4A4_NK_BIG, "flops"),
                             _W4A4NV_SMALL: _bf16_gemm_mean(_W4A4_NK_SMALL, "flops")},
               "extra_counters": ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES"],
               "peak_tflops": 2500.0, "sources": GEMM_SOURCES},
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
    "c3a": {"stem": "mxfp4_absmax_bf16_8192x4096", "kernel": "mxfp4_sweep_kernel",
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
    return [sys.executable, os.path.join(ROOT, "bench.py"), "--config", config, "--steps", str(steps),
            "--warmup", "1", "--no-cpu-baseline", "--copy-calib"]


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
              "VALU issue = SQ_INSTS_VALU x 4 cycles / (SIMDs x trace duration x clock); VALUBusy = "
              "100 x SQ_ACTIVE_INST_VALU / CUs / (GRBM_GUI_ACTIVE / XCDs), the counter runs being "
              "slower than the trace.", "",
              "| kernel | waves | VALU insts | VALU issue | VALUBusy | FETCH KiB | WRITE KiB | HBM bytes "
              "(calibrated) | algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|---|---|---|"]
    record = None
    for name, avg_us in durations.items():
        if not _ours(name):
            continue
        key = _short(name) if _short(name) in w["alg_bytes"] else _short(name).split("<")[0]
        insts = pick(valu, name, "SQ_INSTS_VALU")
        waves = pick(valu, name, "SQ_WAVES")
        active = pick(valu, name, "SQ_ACTIVE_INST_VALU")
        grbm = pick(valu, name, "GRBM_GUI_ACTIVE")
        fk = pick(fetch, name, "FETCH_SIZE")
        wk = pick(write, name, "WRITE_SIZE")
        issue = insts[0] * 4 / (simds * avg_us * 1e-6 * clk_mhz * 1e6) if insts else None
        busy = 100 * active[0] / cus / (grbm[0] / xcc) if active and grbm else None
        hbm = (fk[0] * 1024 * f_factor + wk[0] * 1024 * w_factor) if (fk and wk and f_factor) else None
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
    if w.get("alg_flops"):
        lines += ["", "## Matrix cores", "",
                  f"Achieved = mean algorithmic flops per dispatch / average duration; peak = the published dense "
                  f"FP4 figure ({w['peak_tflops']:.0f} TFLOP/s at 2.4 GHz).  MFMA busy share = "
                  "SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE / XCDs); cycles per MFMA = "
                  "SQ_VALU_MFMA_BUSY_CYCLES / SQ_INSTS_MFMA.", "",
                  "| kernel | flops per dispatch | achieved TFLOP/s | of peak | MFMA insts | cycles per MFMA | "
                  "MFMA busy share | GPU clock (GRBM) |", "|---|---|---|---|---|---|---|---|"]
        for name, avg_us in durations.items():
            fl = w["alg_flops"].get(_short(name))
            if fl is None:
                continue
            mi = pick(valu, name, "SQ_INSTS_MFMA")
            mb = pick(valu, name, "SQ_VALU_MFMA_BUSY_CYCLES")
            grbm = pick(valu, name, "GRBM_GUI_ACTIVE")
            tf = fl / (avg_us * 1e-6) / 1e12
            share = mb[0] / (simds * grbm[0] / xcc) if (mb and grbm) else None
            cpm = mb[0] / mi[0] if (mb and mi and mi[0]) else None
            lines.append(f"| `{_short(name)}` | {fl:.4g} | {tf:.0f} | {100 * tf / w['peak_tflops']:.1f}% | "
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
    a = ap.parse_args()
    if a.cmd == "run":
        run(a.config, a.out, a.steps)
    else:
        summarize(a.config, a.in_dir, a.profiles)


if __name__ == "__main__":
    main()
