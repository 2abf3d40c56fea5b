"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-next]

One step runs the whole hot path once per workload, on inputs already
resident in HBM, one launch per leg:
  * bf16 forward on every 16-bit workload shape: B=2 H=16 N=8192 d=128 causal
    and non-causal (the long-context d=128 regime), B=8 H=16 N=2048 d=128
    non-causal and causal, B=4 H=32 N=4096 d=64 non-causal, B=2 H=8 N=16384
    d=256 causal;
  * the fp8 path on B=4 H=16 N=4096 d=128 (0.1 % outliers): fa_fp8_prep_qkv,
    one launch that prepares Q and K (random-sign Hadamard + 128-row
    power-of-two block scales, Q prescaled by softmax_scale * log2(e)) and V
    (power-of-two block scales), then the fp8 forward in its multiply-free
    form (FA_FP8_QSCALED).
Each leg is timed with HIP events on the stream it is launched on.

Headlines, one per precision (work 4*B*H*N^2*d, halved for causal):
  * value: bf16 forward TFLOP/s at B=2 H=16 N=8192 d=128, causal and
    non-causal launches together (their work over their summed time);
  * headlines.bf16_all: every bf16 leg of the step together;
  * headlines.fp8: the fp8 forward leg, against the dense fp8 peak, and the
    prep + forward pair end to end.
`roofline` is the longest leg of the headline (the non-causal N=8192 launch)
against the dense bf16 MFMA peak; `rooflines` has one entry per forward leg
naming its kernel. Each carries the HBM bytes per launch measured by
rocprofv3 counters when the committed summary was taken on the kernel's
current machine code (else null). `cpu_baseline` times the float64 oracle on
a bounded sample of the same workloads (rank 0, N=1 only).

After the step, the rows built beyond the forward are timed on their own and
reported under `next_rows` (not part of any headline): the 16-bit backward,
the fused rotary + Hadamard + fp8 prep, the microscaled fp8 variant, the
block-scaled fp8 forward causal, the fp8 forward on inputs prepared without
the prescale (amax / 448 scales for Q and K) and the decode-shaped forward
(see build_next_legs).

Prints ONE JSON line on stdout.
"""

import argparse
import hashlib
import json
import os
import struct
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import exact_attention_55_amd as fa  # noqa: E402
from exact_attention_55_amd.inputs import (CONFIGS, DECODE_CONFIGS, attention_flops,  # noqa: E402
                                           make_decode, make_dout, make_qkv, make_signs)

PEAK_BF16 = 2516.6   # TFLOP/s, MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_FP8 = 5033.2    # TFLOP/s, dense fp8
PEAK_HBM = 8000.0    # GB/s

FP8 = "fp8_b4h16n4k_d128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")

# Forward legs of the step: leg name -> (workload, kernel symbol in the code
# object). The kernel is the one the library's launch picks for the shape.
_F16 = "_ZN2fa15fa_fwd16_kernelIDF16bLi{d}ELb{c}ELb0ELb{w}EEEvPKT_S3_S3_PvPfiiif"
# the 64-rows-per-wave pipelined kernel, which the library runs for
# non-causal d = 128 at N >= 8192
_F16P = "_ZN2fa12_GLOBAL__N_120fa_fwd16_pipe_kernelIDF16bLi128ELb0ELb0EEEvPKT_S4_S4_PvPfiiif"
FWD16_LEGS = {
    "bf16_fwd_b2h16n8k_d128_causal": ("b2h16n8k_d128_causal", _F16.format(d=128, c=1, w=0)),
    "bf16_fwd_b2h16n8k_d128": ("b2h16n8k_d128", _F16P),
    "bf16_fwd_b8h16n2k_d128": ("b8h16n2k_d128", _F16.format(d=128, c=0, w=0)),
    "bf16_fwd_b8h16n2k_d128_causal": ("b8h16n2k_d128_causal", _F16.format(d=128, c=1, w=0)),
    "bf16_fwd_b4h32n4k_d64": ("b4h32n4k_d64", _F16.format(d=64, c=0, w=1)),
    "bf16_fwd_b2h8n16k_d256_causal": ("b2h8n16k_d256_causal", _F16.format(d=256, c=1, w=0)),
}
FP8_FWD_LEG = "fp8_fwd_b4h16n4k_d128"
FP8_PREP_LEG = "fp8_prep_qkv_b4h16n4k_d128"
FP8_SYMBOL = "_ZN2fa17fa_fwd_fp8_kernelILi128ELb0ELb0ELb0ELb1EEEvPKhS2_S2_PvPfiiiimf"
KERNEL_OF = {**{k: v[1] for k, v in FWD16_LEGS.items()}, FP8_FWD_LEG: FP8_SYMBOL}
# the HBM-bound kernel of the step (Q, K, V fp8 prep in one launch)
PREP_SYMBOL = "_ZN2fa19fp8_prep_qkv_kernelIDF16bLi128EEEvPKT_S3_S3_PhS4_S4_PKamiiiif"
# kernels whose HBM traffic is measured: the forward legs' and the prep's
TRAFFIC_OF = {**KERNEL_OF, FP8_PREP_LEG: PREP_SYMBOL}
HEADLINE = ["bf16_fwd_b2h16n8k_d128_causal", "bf16_fwd_b2h16n8k_d128"]
ROOF_LEG = "bf16_fwd_b2h16n8k_d128"


def _elf_sections(elf):
    """(name, address, file offset, size) of every section of a little-endian
    ELF64 image, in section-index order."""
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    raw = [struct.unpack_from("<IIQQQQ", elf, shoff + i * shentsize) for i in range(shnum)]
    stroff = raw[shstrndx][4]
    return [(elf[stroff + r[0]:elf.index(b"\0", stroff + r[0])].decode(), r[3], r[4], r[5])
            for r in raw]


def _gfx950_code_objects():
    """The gfx950 code objects inside libfa.so: its .hip_fatbin section holds
    one clang offload bundle per translation unit, each with one code object
    per target."""
    path = os.path.join(ROOT, "exact_attention_55_amd", "libfa.so")
    with open(path, "rb") as f:
        elf = f.read()
    fat = [(o, n) for name, _, o, n in _elf_sections(elf) if name == ".hip_fatbin"]
    if not fat:
        raise RuntimeError(f"no .hip_fatbin section in {path}")
    sec = elf[fat[0][0]:fat[0][0] + fat[0][1]]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    out, start = [], sec.find(magic)
    while start >= 0:
        count, = struct.unpack_from("<Q", sec, start + 24)
        pos = start + 32
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", sec, pos)
            triple = sec[pos + 24:pos + 24 + tlen].decode()
            pos += 24 + tlen
            if triple.endswith("gfx950"):
                out.append(sec[start + off:start + off + size])
        start = sec.find(magic, start + 1)
    if not out:
        raise RuntimeError("no gfx950 code object in the fat binary")
    return out


def source_hash(symbol):
    """SHA-256 of one kernel's machine code in the built library: the bytes of
    its function and of its kernel descriptor (with the position-dependent
    entry offset cleared). It changes exactly when that kernel's compiled
    code changes, not with comments, host code or other kernels."""
    for code in _gfx950_code_objects():
        shdrs = _elf_sections(code)
        secs = {name: (o, n) for name, _, o, n in shdrs}
        symoff, symsize = secs[".symtab"]
        stroff = secs[".strtab"][0]
        h = hashlib.sha256()
        found = 0
        for j in range(symsize // 24):
            st_name, _, _, shndx, value, size = struct.unpack_from("<IBBHQQ", code, symoff + j * 24)
            name = code[stroff + st_name:code.index(b"\0", stroff + st_name)].decode()
            if name not in (symbol, symbol + ".kd") or size == 0:
                continue
            _, addr, soff, _ = shdrs[shndx]
            start = soff + value - addr                # file offset of the symbol
            blob = bytearray(code[start:start + size])
            if name.endswith(".kd"):
                blob[16:24] = bytes(8)                 # kernel_code_entry_byte_offset
            h.update(name.encode() + bytes(blob))
            found += 1
        if found == 2:
            return h.hexdigest()
    raise RuntimeError(f"kernel {symbol} not found in the code objects")


def measured_traffic(leg):
    """HBM bytes per launch of a forward leg's kernel from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain
    copy), or None when that kernel's machine code changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)["legs"][leg]
    except (OSError, ValueError, KeyError):
        return None
    if t.get("code_sha256") != source_hash(TRAFFIC_OF[leg]):
        return None
    return t.get("hbm_bytes_per_launch")


def algorithmic_bytes(leg):
    """Bytes a kernel must move per launch. Forward: Q, K, V in, O out, LSE
    out (and the fp8 scales). fp8 prep: the three 16-bit tensors in, their
    codes and block scales out."""
    if leg == FP8_PREP_LEG:
        c = CONFIGS[FP8]
        nel = c["B"] * c["H"] * c["N"] * c["d"]
        return 3 * (2 * nel + nel + 4 * c["B"] * c["H"] * ((c["N"] + 127) // 128))
    if leg == FP8_FWD_LEG:
        c = CONFIGS[FP8]
        nel = c["B"] * c["H"] * c["N"] * c["d"]
        rows = c["B"] * c["H"] * c["N"]
        return 3 * nel + 2 * nel + 4 * rows + 3 * 4 * c["B"] * c["H"] * (c["N"] // 128)
    c = CONFIGS[FWD16_LEGS[leg][0]]
    nel = c["B"] * c["H"] * c["N"] * c["d"]
    return 4 * nel * 2 + 4 * c["B"] * c["H"] * c["N"]


def traffic_commands():
    cmds = []
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        for leg in TRAFFIC_OF:
            cmds.append(f"rocprofv3 --pmc {c} -d <out>/pmc_{c} -o {leg} -f csv -- python3 bench.py "
                        f"--only {leg} --steps 3 --warmup 1 --no-cpu --no-next")
        cmds.append(f"rocprofv3 --pmc {c} -d <out>/pmc_{c} -o copy -f csv -- python3 bench.py --copy-calib")
    return cmds + ["python3 bench.py --traffic-summary <out>"]


def traffic_summary(run_dir):
    """Write TRAFFIC_FILE from the counter runs under run_dir (see
    traffic_commands): per forward leg, FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch of its kernel) each scaled by what the same counter reads for a
    plain 1 GiB device copy."""
    import csv

    def per_dispatch(path, name_part):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if name_part in r["Kernel_Name"]:
                    vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return vals

    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = per_dispatch(os.path.join(run_dir, f"pmc_{c}", "copy_counter_collection.csv"), "")
        copy_kib = sorted(copy.values())[-2]          # median of the three 1 GiB copies
        scale[c] = {"copy_kib": copy_kib, "scale": (1 << 30) / 1024.0 / copy_kib}
    legs = {}
    for leg, sym in TRAFFIC_OF.items():
        part = _short_kernel_name(sym).split("<")[0]
        e = {"kernel_symbol": sym}
        try:
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                v = per_dispatch(os.path.join(run_dir, f"pmc_{c}", f"{leg}_counter_collection.csv"), part)
                kib = float(np.mean(list(v.values())))
                e[c] = {"kib_per_dispatch": kib, "dispatches": len(v),
                        "bytes_per_launch": kib * 1024 * scale[c]["scale"]}
        except (OSError, ValueError):
            continue
        e["hbm_bytes_per_launch"] = e["FETCH_SIZE"]["bytes_per_launch"] + e["WRITE_SIZE"]["bytes_per_launch"]
        e["algorithmic_bytes_per_launch"] = algorithmic_bytes(leg)
        e["traffic_over_algorithmic"] = e["hbm_bytes_per_launch"] / e["algorithmic_bytes_per_launch"]
        e["code_sha256"] = source_hash(sym)
        legs[leg] = e
    summary = {"commands": traffic_commands(), "copy_calibration": scale, "legs": legs}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(summary, f, indent=1)
    print(json.dumps(summary, indent=1))


TRACE_FILE = os.path.join(ROOT, "profiles", "bench_kernel_trace.md")


def trace_commands():
    """The kernel-trace run of the whole bench (from the repository root;
    <out> a scratch directory)."""
    return ["rocprofv3 --kernel-trace --stats -d <out>/trace_all -o run -f csv -- python3 bench.py "
            "--steps 5 --warmup 2 --no-cpu",
            "python3 bench.py --trace-summary <out>"]


def _short_kernel_name(n):
    """Kernel name with its template arguments, from the mangled symbol (the
    demangler leaves the bf16 ones mangled) or the demangled form."""
    import re
    import subprocess
    m = re.match(r"_ZN2fa(?:12_GLOBAL__N_1)?(\d+)", n)
    if m:
        k = int(m.group(1))
        rest = n[m.end():]
        name, rest = rest[:k], rest[k:]
        if rest.startswith("I") and "EEv" in rest:
            toks = re.findall(r"(DF16b)|(DF16_)|Li(\d+)E|Lb([01])E", rest[1:rest.index("EEv") + 1])
            args = ["bf16" if a else "fp16" if b else c if c else ("true" if d == "1" else "false")
                    for a, b, c, d in toks]
            return f"{name}<{','.join(args)}>"
        return name
    try:
        n = subprocess.run(["c++filt", n], capture_output=True, text=True).stdout.strip() or n
    except OSError:
        pass
    n = n.replace("fa::(anonymous namespace)::", "").replace("fa::", "").replace("void ", "")
    return n.split("(")[0].replace("__bf16", "bf16").replace(" ", "")


def trace_summary(run_dir, warmup=2, steps=5):
    """Write TRACE_FILE from the run of trace_commands under run_dir. Per
    forward leg: its kernel's dispatches in the timed steps. Every step runs
    the legs in order, one dispatch of its kernel each, so the dispatches of
    a kernel that several legs share go to those legs in turn."""
    import csv
    base = os.path.join(run_dir, "trace_all")
    with open(os.path.join(base, "run_kernel_trace.csv")) as f:
        trace = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    lines = ["# Kernel trace of bench.py", "",
             "Commands (repository root, TMPDIR=/tmp, <out> a scratch directory):", ""]
    lines += ["    " + c for c in trace_commands()]
    lines += ["", f"## Forward legs of the step ({steps} timed steps after {warmup} warm-up ones)", "",
              "| leg | kernel | dispatches | avg us | min us | max us | TFLOP/s at avg | of peak |",
              "|---|---|---|---|---|---|---|---|"]
    order = list(KERNEL_OF)
    for leg, sym in KERNEL_OF.items():
        short = _short_kernel_name(sym)
        sharing = [l for l in order if _short_kernel_name(KERNEL_OF[l]) == short]
        disp = [r for r in trace if r["Kernel_Name"] == sym or _short_kernel_name(r["Kernel_Name"]) == short]
        disp = disp[: (warmup + steps) * len(sharing)]
        mine = disp[sharing.index(leg)::len(sharing)][warmup:]
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in mine]
        if not d:
            continue
        if leg == FP8_FWD_LEG:
            c, peak = CONFIGS[FP8], PEAK_FP8
        else:
            c, peak = CONFIGS[FWD16_LEGS[leg][0]], PEAK_BF16
        fl = attention_flops(c["B"], c["H"], c["N"], c["d"], c["causal"])
        avg = float(np.mean(d))
        lines.append(f"| {leg} | {short} | {len(d)} | {avg:.1f} | {min(d):.1f} | {max(d):.1f} | "
                     f"{fl / avg / 1e6:.0f} | {fl / avg / 1e6 / peak:.3f} |")
    with open(os.path.join(base, "run_kernel_stats.csv")) as f:
        rows = list(csv.DictReader(f))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    lines += ["", "## All kernels of the run (step legs, then the rows beyond the forward)", "",
              "A kernel several legs share is averaged over all of them here.", "",
              "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {_short_kernel_name(r['Name'])} | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / tot * 100:.1f} |")
    text = "\n".join(lines) + "\n"
    with open(TRACE_FILE, "w") as f:
        f.write(text)
    print(text)


# Ablations of the 16-bit forward: variant -> (build.py -D flags or None for
# the default library, leg-name suffix). Each is measured on the two d = 128
# workloads below with two SQ counter passes.
ABLATIONS = {
    "default": (None, ""),
    "pingpong": (["-DFA16_PINGPONG=1"], ""),
    "no_setprio": (["-DFA16_PRIO=0"], ""),
    "compiler_schedule": (["-DFA16_SCHED=0"], ""),
    "read_ahead_2": (["-DFA16_KPD=2", "-DFA16_VPD=2"], ""),
    "eight_waves": (["-DFA16_CFG_128=8,1,64,2"], ""),
    "pipelined_64_rows": (None, "_pipelined"),
    "fp8_default": (None, "fp8"),          # the fp8 forward's counters
    "fp8_unpinned_scores": (["-DFA8_KEEP=0"], "fp8"),
    "fp8_multiply_per_score": (["-DFA8_QS=0"], "fp8"),
    "fp8_exact_reference": (["-DFA8_MARGIN=0.0f"], "fp8"),
    "fp8_barrier_per_tile": (["-DFA8_PAIRSYNC=0"], "fp8"),
}
ABLATION_LEGS = ["bf16_fwd_b8h16n2k_d128", "bf16_fwd_b2h16n8k_d128_causal"]


def _ablation_legs(suffix):
    """The legs of one ablation run, in the order build_legs runs them."""
    if suffix == "fp8":
        return [FP8_FWD_LEG]
    order = list(FWD16_LEGS)
    return [leg + suffix for leg in sorted(ABLATION_LEGS, key=order.index)]
COUNTER_PASSES = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
    "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE",
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_MISC SQ_WAIT_INST_LDS SQ_LDS_IDX_ACTIVE "
    "SQ_WAIT_ANY SQ_INSTS_SALU SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE",
]
ABLATION_FILE = os.path.join(ROOT, "profiles", "ablation_fwd16_d128.md")


def ablation_commands():
    """Build and counter commands of the ablation table (from the repository
    root; <out> a scratch directory)."""
    cmds = []
    for name, (flags, suffix) in ABLATIONS.items():
        lib = ""
        if flags:
            cmds.append(f"python3 -m exact_attention_55_amd.build --variant {name} " + " ".join(flags))
            lib = f"FA_LIB=exact_attention_55_amd/variants/libfa_{name}.so "
        only = " ".join(f"--only {leg}" for leg in _ablation_legs(suffix))
        for i, ctr in enumerate(COUNTER_PASSES):
            cmds.append(f"{lib}rocprofv3 --pmc {ctr} -d <out>/{name}_p{i + 1} -o run -f csv -- "
                        f"python3 bench.py {only} --steps 3 --warmup 1 --no-cpu --no-next")
    return cmds + ["python3 bench.py --counter-summary <out>"]


def counter_summary(run_dir):
    """Write ABLATION_FILE from the counter runs under run_dir (see
    ablation_commands): per variant and workload, the mean per dispatch of
    each counter over the forward kernel's dispatches, and the derived
    figures."""
    import csv
    rows = []
    for name, (_, suffix) in ABLATIONS.items():
        legs = _ablation_legs(suffix)
        per = {}
        for i in range(len(COUNTER_PASSES)):
            path = os.path.join(run_dir, f"{name}_p{i + 1}", "run_counter_collection.csv")
            disp = {}
            with open(path) as f:
                for r in csv.DictReader(f):
                    if "fa_fwd" not in r["Kernel_Name"]:
                        continue
                    d = disp.setdefault(int(r["Dispatch_Id"]), {})
                    d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            # every step runs the legs in order, one forward dispatch each
            for k, did in enumerate(sorted(disp)):
                acc = per.setdefault(legs[k % len(legs)], {})
                for c, v in disp[did].items():
                    acc.setdefault(c, []).append(v)
        for leg in legs:
            if leg not in per:
                continue
            m = {c: float(np.mean(v)) for c, v in per[leg].items()}
            cyc = m["GRBM_GUI_ACTIVE"] / 8                # per XCD
            waves = m["SQ_WAVES"]
            rows.append((name, leg, {
                "cycles": cyc,
                "mfma_busy": m["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cyc),
                "valu_active": m["SQ_ACTIVE_INST_VALU"] / m["SQ_WAVE_CYCLES"],
                "wait_any": m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"],
                "wait_lds": m["SQ_WAIT_INST_LDS"] / m["SQ_WAVE_CYCLES"],
                "valu_per_wave": m["SQ_INSTS_VALU"] / waves,
                "mfma_per_wave": m["SQ_INSTS_MFMA"] / waves,
                "lds_per_wave": m["SQ_INSTS_LDS"] / waves,
                "bank_conflicts": m["SQ_LDS_BANK_CONFLICT"],
            }))
    lines = ["# Ablations of the 16-bit and fp8 forwards at d = 128 (SQ counters)", "",
             "Each variant is a compile-time switch of `csrc/fa_fwd16.hip` (FA16_*) or",
             "`csrc/fa_fwd_fp8.hip` (FA8_*) built with",
             "`python3 -m exact_attention_55_amd.build --variant NAME -D...` and loaded through",
             "`FA_LIB`; `pipelined_64_rows` is the default library with `FA_FWD_PIPELINED`.",
             "Commands (repository root, TMPDIR=/tmp, <out> a scratch directory):", ""]
    lines += ["    " + c for c in ablation_commands()]
    lines += ["", "Mean per dispatch over the kernel's dispatches (3 timed + 1 warm-up). cycles: "
              "GRBM_GUI_ACTIVE / 8 (one XCD); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x "
              "cycles); VALU active and waits are fractions of SQ_WAVE_CYCLES; instruction counts "
              "per wave.", "",
              "| variant | workload | cycles | MFMA busy | VALU active | wait any | wait LDS | "
              "VALU / wave | MFMA / wave | LDS / wave | bank conflicts |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, leg, v in rows:
        lines.append(f"| {name} | {leg} | {v['cycles']:.3g} | {100 * v['mfma_busy']:.1f} % | "
                     f"{100 * v['valu_active']:.1f} % | {100 * v['wait_any']:.1f} % | "
                     f"{100 * v['wait_lds']:.1f} % | {v['valu_per_wave']:.0f} | "
                     f"{v['mfma_per_wave']:.0f} | {v['lds_per_wave']:.0f} | {v['bank_conflicts']:.0f} |")
    text = "\n".join(lines) + "\n"
    with open(ABLATION_FILE, "w") as f:
        f.write(text)
    print(text)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Leg:
    def __init__(self, name, fn, flops=0.0, bytes_=0.0, peak=PEAK_BF16):
        self.name, self.fn, self.flops, self.bytes, self.peak = name, fn, flops, bytes_, peak
        self.times = []

    def run(self, timed):
        if timed:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            self.fn()
            b.record()
            return (a, b)
        self.fn()
        return None


def build_legs(dev, only=None):
    """The step's legs (all, or the names in `only`) and the tensors they use.
    With `only`, a 16-bit forward leg's name plus "_pipelined" selects the
    same leg run by the 64-rows-per-wave pipelined kernel (an ablation)."""
    legs, keep = [], []
    names = [(n, False) for n in FWD16_LEGS]
    if only:
        names += [(n, True) for n in FWD16_LEGS if n + "_pipelined" in only]
    for name, piped in names:
        cfg = FWD16_LEGS[name][0]
        if only and not piped and name not in only:
            continue
        c = CONFIGS[cfg]
        q, k, v = (t.to(dev) for t in make_qkv(**c))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        fl = attention_flops(c["B"], c["H"], c["N"], c["d"], c["causal"])
        legs.append(Leg(name + ("_pipelined" if piped else ""),
                        lambda q=q, k=k, v=v, o=o, lse=lse, causal=c["causal"], piped=piped:
                        fa.fwd(q, k, v, causal, out=o, lse=lse, pipelined=piped), fl))
        keep += [q, k, v, o, lse]
    if only and FP8_PREP_LEG not in only and FP8_FWD_LEG not in only:
        return legs, keep
    c8 = CONFIGS[FP8]
    B8, H8, N8, d8 = c8["B"], c8["H"], c8["N"], c8["d"]
    q8, k8, v8 = (t.to(dev) for t in make_qkv(**c8))
    signs = torch.from_numpy(make_signs(H8, d8, c8["seed"])).to(dev)
    pq, pk, pv = (fa.fp8_alloc_packed(B8, H8, N8, d8, dev) for _ in range(3))
    o8 = torch.empty((B8, H8, N8, d8), dtype=torch.bfloat16, device=dev)
    lse8 = torch.empty((B8, H8, N8), dtype=torch.float32, device=dev)
    nel = B8 * H8 * N8 * d8
    prep_bytes = 3 * (nel * 2 + nel + B8 * H8 * (N8 // 128) * 4)

    prescale = fa.qk_prescale(1.0 / d8 ** 0.5)

    def prep():
        fa.fp8_prep_qkv(q8, k8, v8, signs, q_prescale=prescale, out=(pq, pk, pv))

    prep()                      # the forward leg alone still reads prepared inputs
    if not only or FP8_PREP_LEG in only:
        legs.append(Leg(FP8_PREP_LEG, prep, 0.0, prep_bytes))
    if not only or FP8_FWD_LEG in only:
        legs.append(Leg(FP8_FWD_LEG,
                        lambda: fa.fwd_fp8(pq, pk, pv, B8, H8, N8, d8, False, out=o8, lse=lse8,
                                           qscaled=True),
                        attention_flops(B8, H8, N8, d8, False), peak=PEAK_FP8))
    keep += [q8, k8, v8, signs, pq, pk, pv, o8, lse8]
    return legs, keep


def build_next_legs(dev):
    """Legs of the rows beyond the forward; timed apart from the step:
    the 16-bit backward (dQ, dK, dV from the saved LSE) on B=8 H=16 N=2048
    d=128, work 10*B*H*N^2*d (the five GEMMs of the gradient, halved for
    causal); the fused rotary + Hadamard + fp8 block quantisation of Q and K
    of the fp8 workload (half pairing, GB/s of bytes read and written); the
    microscaled fp8 variant (fa_mx_prep_qkv: Q, K along d with the Hadamard,
    Q prescaled, and V along the sequence in one launch, GB/s, and the same
    as three fa_mx_prep calls; the forward on its output, non-causal and
    causal); the block-scaled fp8 forward, causal; the fp8
    forward on inputs prepared without the prescale (amax / 448 scales for Q
    and K, one multiply-add per score); the step's fp8 prep as three
    separate fa_fp8_prep calls (GB/s); and the decode-shaped
    forward on its two workloads, in GB/s of the bytes it must move (K and V
    of every sequence's keys, Q, O, LSE); the backward at d = 256 on the
    B=2 H=8 N=16384 causal workload; and, as an ablation, the pipelined
    16-bit kernel on the causal B=2 H=16 N=8192 workload (the step already
    runs it on the non-causal one)."""
    legs = []
    c = CONFIGS["b8h16n2k_d128"]
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    q, k, v = (t.to(dev) for t in make_qkv(**c))
    do = make_dout(B, H, N, d, c["seed"] + 500, c["dtype"]).to(dev)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    delta = torch.empty((2, B, H, N), dtype=torch.float32, device=dev)
    keep = [q, k, v, do, grads, delta]
    for causal in (False, True):
        o, lse = fa.fwd(q, k, v, causal)
        keep += [o, lse]
        fl = 2.5 * attention_flops(B, H, N, d, causal)
        name = "bf16_bwd_b8h16n2k_d128" + ("_causal" if causal else "")
        legs.append(Leg(name, lambda o=o, lse=lse, causal=causal: fa.bwd(
            q, k, v, o, lse, do, causal, grads=grads, delta=delta), fl))
    # the 64-rows-per-wave pipelined kernel (FA_FWD_PIPELINED) on the causal
    # 16-bit headline workload, beside the default kernel the step times
    for cfg in ("b2h16n8k_d128_causal",):
        cp = CONFIGS[cfg]
        qp, kp, vp = (t.to(dev) for t in make_qkv(**cp))
        op = torch.empty_like(qp)
        lp = torch.empty(qp.shape[:3], dtype=torch.float32, device=dev)
        keep += [qp, kp, vp, op, lp]
        legs.append(Leg("bf16_fwd_" + cfg + "_pipelined",
                        lambda qp=qp, kp=kp, vp=vp, op=op, lp=lp, causal=cp["causal"]:
                        fa.fwd(qp, kp, vp, causal, out=op, lse=lp, pipelined=True),
                        attention_flops(cp["B"], cp["H"], cp["N"], cp["d"], cp["causal"])))
    # the backward at d = 256 on the long-sequence d = 256 forward workload
    c4 = CONFIGS["b2h8n16k_d256_causal"]
    q4, k4, v4 = (t.to(dev) for t in make_qkv(**c4))
    do4 = make_dout(c4["B"], c4["H"], c4["N"], c4["d"], c4["seed"] + 500, c4["dtype"]).to(dev)
    o4, l4 = fa.fwd(q4, k4, v4, True)
    g4 = tuple(torch.empty_like(q4) for _ in range(3))
    dl4 = torch.empty((2,) + tuple(q4.shape[:3]), dtype=torch.float32, device=dev)
    keep += [q4, k4, v4, do4, o4, l4, g4, dl4]
    legs.append(Leg("bf16_bwd_b2h8n16k_d256_causal", lambda: fa.bwd(
        q4, k4, v4, o4, l4, do4, True, grads=g4, delta=dl4),
        2.5 * attention_flops(c4["B"], c4["H"], c4["N"], c4["d"], True)))
    c8 = CONFIGS[FP8]
    B8, H8, N8, d8 = c8["B"], c8["H"], c8["N"], c8["d"]
    q8, k8, v8 = (t.to(dev) for t in make_qkv(**c8))
    signs = torch.from_numpy(make_signs(H8, d8, c8["seed"])).to(dev)
    pq, pk = (fa.fp8_alloc_packed(B8, H8, N8, d8, dev) for _ in range(2))
    nel = B8 * H8 * N8 * d8
    rope_bytes = 2 * (nel * 2 + nel + B8 * H8 * (N8 // 128) * 4)

    def prep_rope():
        fa.fp8_prep(q8, signs, 128, out=pq, rope=("half", 10000.0, 0))
        fa.fp8_prep(k8, signs, 128, out=pk, rope=("half", 10000.0, 0))

    legs.append(Leg("fp8_prep_rope_qk_b4h16n4k_d128", prep_rope, 0.0, rope_bytes))
    keep += [q8, k8, v8, signs, pq, pk]
    mq, mk, mv = (torch.empty(fa.mx_packed_bytes(B8, H8, N8, d8), dtype=torch.uint8, device=dev)
                  for _ in range(3))
    mx_bytes = 3 * (nel * 2 + nel + nel // 32)

    prescale = fa.qk_prescale(1.0 / d8 ** 0.5)

    def prep_mx():
        fa.mx_prep_qkv(q8, k8, v8, signs, q_prescale=prescale, out=(mq, mk, mv))

    def prep_mx_separate():
        fa.mx_prep(q8, signs, "d", out=mq, prescale=prescale)
        fa.mx_prep(k8, signs, "d", out=mk)
        fa.mx_prep(v8, None, "n", out=mv)

    legs.append(Leg("fp8_mx_prep_qkv_b4h16n4k_d128", prep_mx, 0.0, mx_bytes))
    legs.append(Leg("fp8_mx_prep_qkv_separate_b4h16n4k_d128", prep_mx_separate, 0.0, mx_bytes))
    prep_mx()
    o8 = torch.empty((B8, H8, N8, d8), dtype=torch.bfloat16, device=dev)
    lse8 = torch.empty((B8, H8, N8), dtype=torch.float32, device=dev)
    for causal in (False, True):
        legs.append(Leg("fp8_mx_fwd_b4h16n4k_d128" + ("_causal" if causal else ""),
                        lambda causal=causal: fa.fwd_fp8(mq, mk, mv, B8, H8, N8, d8, causal, out=o8,
                                                         lse=lse8, mx=True, qscaled=True),
                        attention_flops(B8, H8, N8, d8, causal), peak=PEAK_FP8))
    keep += [mq, mk, mv, o8, lse8]
    bq = fa.fp8_prep(q8, signs, 128, prescale=prescale)
    bk = fa.fp8_prep(k8, signs, 128, pow2_scale=True)
    bv = fa.fp8_prep(v8, None, 128, pow2_scale=True)
    legs.append(Leg("fp8_fwd_b4h16n4k_d128_causal",
                    lambda: fa.fwd_fp8(bq, bk, bv, B8, H8, N8, d8, True, out=o8, lse=lse8,
                                       qscaled=True),
                    attention_flops(B8, H8, N8, d8, True), peak=PEAK_FP8))
    uq, uk = (fa.fp8_prep(t, signs, 128) for t in (q8, k8))

    def prep_separate():
        fa.fp8_prep(q8, signs, 128, out=bq, prescale=prescale)
        fa.fp8_prep(k8, signs, 128, out=bk, pow2_scale=True)
        fa.fp8_prep(v8, None, 128, out=bv, pow2_scale=True)

    legs.append(Leg("fp8_prep_qkv_separate_b4h16n4k_d128", prep_separate, 0.0,
                    3 * (nel * 2 + nel + B8 * H8 * (N8 // 128) * 4)))
    legs.append(Leg("fp8_fwd_b4h16n4k_d128_unscaled",
                    lambda: fa.fwd_fp8(uq, uk, bv, B8, H8, N8, d8, False, out=o8, lse=lse8),
                    attention_flops(B8, H8, N8, d8, False), peak=PEAK_FP8))
    keep += [bq, bk, bv, uq, uk]
    for name, c in sorted(DECODE_CONFIGS.items()):
        B, H, Hkv, Nq, Nk, d = c["B"], c["H"], c["Hkv"], c["Nq"], c["Nk"], c["d"]
        qh, kh, vh, sl = make_decode(**c)
        qd, kd, vd = (t.to(dev) for t in (qh, kh, vh))
        sld = None if sl is None else sl.to(dev)
        splits = fa.decode_splits(B, H, Hkv, Nq, Nk, d)
        ws = torch.empty(max(1, fa.decode_workspace_bytes(B, H, Nq, d, splits)), dtype=torch.uint8,
                         device=dev)
        od = torch.empty((B, H, Nq, d), dtype=qd.dtype, device=dev)
        ld = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
        keys = Nk * B if sl is None else int(sl.sum())
        nbytes = keys * Hkv * d * 2 * 2 + 2 * B * H * Nq * d * 2 + 4 * B * H * Nq
        legs.append(Leg("bf16_" + name, lambda qd=qd, kd=kd, vd=vd, sld=sld, od=od, ld=ld, ws=ws,
                        s=splits, causal=c["causal"]: fa.fwd_decode(
                            qd, kd, vd, causal, seqlens_k=sld, num_splits=s, out=od, lse=ld,
                            workspace=ws), 0.0, nbytes))
        keep += [qd, kd, vd, sld, od, ld, ws]
    return legs, keep


def time_legs(legs, steps, warmup):
    """Warm up, then time `steps` rounds of every leg; returns the wall time."""
    for _ in range(warmup):
        for L in legs:
            L.run(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    events = [[L.run(True) for L in legs] for _ in range(steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for step in events:
        for L, (a, b) in zip(legs, step):
            L.times.append(a.elapsed_time(b) * 1e-3)
    return wall


def leg_summary(L):
    t = float(np.mean(L.times))
    e = {"ms": t * 1e3, "ms_min": float(np.min(L.times)) * 1e3}
    if L.name == FP8_PREP_LEG:
        e["traffic"] = measured_traffic(L.name)
    if L.flops:
        e["tflops"] = L.flops / t / 1e12
        e["frac_of_peak"] = e["tflops"] / L.peak
    if L.bytes:
        e["gbps"] = L.bytes / t / 1e9
        e["frac_of_hbm"] = e["gbps"] / PEAK_HBM
    return e


def roofline(L):
    t = float(np.mean(L.times))
    achieved = L.flops / t / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": L.peak, "unit": "TFLOP/s",
            "frac": achieved / L.peak, "traffic": measured_traffic(L.name),
            "kernel": KERNEL_OF[L.name], "leg": L.name, "launch_ms": t * 1e3}


def headline(legs):
    fl = sum(L.flops for L in legs)
    t = sum(float(np.mean(L.times)) for L in legs)
    peak = legs[0].peak
    return {"tflops": fl / t / 1e12, "frac_of_peak": fl / t / 1e12 / peak, "peak": peak,
            "legs": [L.name for L in legs], "ms": t * 1e3}


def cpu_baseline():
    """The float64 oracle on a bounded sample of the step's workloads (about
    15-25 s on 16 host cores), on the same seeded inputs: batch 0 (16 heads)
    of B=2 H=16 N=8192 d=128, causal and non-causal (the oracle computes every
    score and masks; the metric counts half for causal), and the fp8 leg as
    the fake-quant oracle (random-sign Hadamard + per-128-row e4m3
    quantisation of the outlier inputs with Q prescaled and power-of-two
    scales, then exact attention) on batch 0 of B=4 H=16 N=4096 d=128. Value:
    the sample's metric flops over the oracle's time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    c, c8 = CONFIGS["b2h16n8k_d128"], CONFIGS[FP8]
    q, k, v = (t[:1].to(torch.float64).numpy() for t in make_qkv(**c))
    q8, k8, v8 = (t[:1].to(torch.float64).numpy() for t in make_qkv(**c8))
    signs = make_signs(c8["H"], c8["d"], c8["seed"])
    fl = (attention_flops(1, c["H"], c["N"], c["d"], False)
          + attention_flops(1, c["H"], c["N"], c["d"], True)
          + attention_flops(1, c8["H"], c8["N"], c8["d"], False))
    t0 = time.perf_counter()
    oracle.attention(q, k, v, False)
    oracle.attention(q, k, v, True)
    oracle.fake_quant_attention(q8, k8, v8, signs, 128, False, prescaled=True)
    el = time.perf_counter() - t0
    return {"value": fl / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"bf16 B=1 (of 2) H=16 N=8192 d=128 non-causal and causal; fp8 fake-quant "
                      f"(Hadamard + block e4m3, Q prescaled) B=1 (of 4) H=16 N=4096 d=128 outlier inputs; "
                      f"float64 numpy oracle, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the rows beyond the forward (backward, rotary prep, decode)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy three times (HBM counter calibration)")
    ap.add_argument("--only", action="append", metavar="LEG",
                    help="only launch these step legs (for counter runs)")
    ap.add_argument("--source-hash", metavar="LEG", help="print a forward leg's kernel code hash")
    ap.add_argument("--traffic-summary", metavar="DIR",
                    help="write the HBM-traffic summary from the counter runs under DIR (no GPU)")
    ap.add_argument("--traffic-commands", action="store_true",
                    help="print the commands of the HBM-traffic counter runs")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="write the kernel-trace summary from the runs under DIR (no GPU)")
    ap.add_argument("--trace-commands", action="store_true",
                    help="print the commands of the kernel-trace runs")
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="write the ablation counter table from the runs under DIR (no GPU)")
    ap.add_argument("--ablation-commands", action="store_true",
                    help="print the commands of the ablation counter runs")
    args = ap.parse_args()
    if args.traffic_commands:
        print("\n".join(traffic_commands()))
        return
    if args.trace_commands:
        print("\n".join(trace_commands()))
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.ablation_commands:
        print("\n".join(ablation_commands()))
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.source_hash:
        print(source_hash(KERNEL_OF[args.source_hash]))
        return
    if args.traffic_summary:
        traffic_summary(args.traffic_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over heads with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calib:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel() * 4, "copies": 3}))
        return
    fa.lib()
    log("building inputs")
    legs, _keep = build_legs(dev, args.only)
    if not legs:
        sys.exit(f"no step leg named {args.only}")
    log(f"timing {args.steps} steps of {len(legs)} legs")
    wall = time_legs(legs, args.steps, args.warmup)
    by = {L.name: L for L in legs}
    out = {
        "metric": "attention fwd TFLOP/s (4*B*H*N^2*d, /2 causal), % of MFMA peak",
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 fwd B=2 H=16 N=8192 d=128, causal + non-causal launches",
                   "global_batch": 2, "seq_len": 8192, "head_dim": 128, "heads": 16,
                   "parallelism": "single-gpu"},
        "legs": {L.name: leg_summary(L) for L in legs},
    }
    if all(n in by for n in HEADLINE):
        h = headline([by[n] for n in HEADLINE])
        out["value"] = h["tflops"]
        out["frac_of_peak"] = h["frac_of_peak"]
        heads = {"bf16_d128_n8k": h}
        bf = [L for L in legs if L.name in FWD16_LEGS]
        heads["bf16_all"] = headline(bf)
        if FP8_FWD_LEG in by:
            f = headline([by[FP8_FWD_LEG]])
            if FP8_PREP_LEG in by:
                tp = float(np.mean(by[FP8_PREP_LEG].times))
                f["with_prep_tflops"] = by[FP8_FWD_LEG].flops / (f["ms"] * 1e-3 + tp) / 1e12
            heads["fp8"] = f
        out["headlines"] = heads
    fwd_legs = [L for L in legs if L.name in KERNEL_OF]
    if ROOF_LEG in by:
        out["roofline"] = roofline(by[ROOF_LEG])
    out["rooflines"] = {L.name: roofline(L) for L in fwd_legs}
    if not args.only and not args.no_next:
        log("timing the rows beyond the forward")
        nlegs, _nkeep = build_next_legs(dev)
        time_legs(nlegs, args.steps, args.warmup)
        out["next_rows"] = {L.name: leg_summary(L) for L in nlegs}
    if not args.only and not args.no_cpu:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
