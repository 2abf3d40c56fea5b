"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-next]

One step runs the whole hot path once, on inputs already resident in HBM:
  1. bf16 forward, B=8 H=16 N=2048 d=128, non-causal   (16k tokens, hidden 2048)
  2. bf16 forward, same shape, causal
  3. fp8 path on B=4 H=16 N=4096 d=128 (0.1% outliers): fa_fp8_prep of Q and K
     (random-sign Hadamard + 128-row block scales) and V (block scales), then
     the fp8 forward.
`value` is the metric work of the step (4*B*H*N^2*d per forward, halved for
causal) divided by the step time. Every leg is also timed on its own with HIP
events on the stream it runs on; `legs` reports each. `roofline` is for the
dominant kernel, the non-causal bf16 forward, against the MI355X dense bf16
MFMA peak. `cpu_baseline` times the float64 oracle on a bounded sample of the
same workload (rank 0, N=1 only).

After the step, the rows built beyond the forward are timed on their own with
the same events and reported under `next_rows` (not part of `value`): the
16-bit backward (dQ, dK, dV from the saved LSE) on the main shape, its work
counted as 10*B*H*N^2*d (the five GEMMs of the gradient, halved for causal);
the fused rotary + Hadamard + fp8 block quantisation of Q and K of the fp8
workload (half pairing, GB/s of bytes read and written); the microscaled fp8
variant on the fp8 workload (fa_mx_prep of Q, K along d with the Hadamard
and V along the sequence, GB/s; the forward on its output, non-causal and
causal, TFLOP/s against the dense fp8 peak); the block-scaled fp8 forward,
causal; and the
decode-shaped forward on its two workloads (B=8 H=16 sequences of
16384 keys; B=16 with 64 query heads over 8 key/value heads and ragged key
counts), in GB/s of the bytes it must move (K and V of every sequence's keys,
Q, O, LSE) against the HBM peak.

Prints ONE JSON line on stdout.
"""

import argparse
import hashlib
import json
import math
import os
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

MAIN = "b8h16n2k_d128"
FP8 = "fp8_b4h16n4k_d128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd16_b8h16n2k_d128_traffic.json")


MAIN_SYMBOL = "_ZN2fa15fa_fwd16_kernelIDF16bLi128ELb0ELb0ELb0EEEvPKT_S3_S3_PvPfiiif"


def _elf_sections(elf):
    """(name, address, file offset, size) of every section of a little-endian
    ELF64 image, in section-index order."""
    import struct
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    raw = [struct.unpack_from("<IIQQQQ", elf, shoff + i * shentsize) for i in range(shnum)]
    stroff = raw[shstrndx][4]
    return [(elf[stroff + r[0]:elf.index(b"\0", stroff + r[0])].decode(), r[3], r[4], r[5])
            for r in raw]


def source_hash(symbol=MAIN_SYMBOL):
    """SHA-256 of one kernel's machine code in the built library: the bytes of
    its function and of its kernel descriptor (with the position-dependent
    entry offset cleared), taken from the gfx950 code object inside the
    .hip_fatbin section of libfa.so. It changes exactly when that kernel's
    compiled code changes, not with comments, host code or other kernels."""
    import struct
    path = os.path.join(ROOT, "exact_attention_55_amd", "libfa.so")
    with open(path, "rb") as f:
        elf = f.read()
    fat = [(o, n) for name, _, o, n in _elf_sections(elf) if name == ".hip_fatbin"]
    if not fat:
        raise RuntimeError(f"no .hip_fatbin section in {path}")
    bundle = elf[fat[0][0]:fat[0][0] + fat[0][1]]
    count, = struct.unpack_from("<Q", bundle, 24)          # clang offload bundle
    pos, code = 32, None
    for _ in range(count):
        off, size, tlen = struct.unpack_from("<QQQ", bundle, pos)
        triple = bundle[pos + 24:pos + 24 + tlen].decode()
        pos += 24 + tlen
        if triple.endswith("gfx950"):
            code = bundle[off:off + size]
    if code is None:
        raise RuntimeError("no gfx950 code object in the fat binary")
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
    if found != 2:
        raise RuntimeError(f"kernel {symbol} not found in the code object")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or
    None when the kernels changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("code_sha256") != source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def traffic_summary(run_dir):
    """Build the HBM-traffic summary of the dominant kernel from four
    rocprofv3 counter runs under run_dir (pmc_FETCH_SIZE/{main,copy} and
    pmc_WRITE_SIZE/{main,copy}, see TRAFFIC_COMMANDS) and write it to
    TRAFFIC_FILE. FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by
    what the same counter reads for a plain 1 GiB device copy."""
    import csv

    def per_dispatch(path, name_part):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if name_part in r["Kernel_Name"]:
                    vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return vals

    out = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        main = per_dispatch(os.path.join(run_dir, f"pmc_{c}", "main_counter_collection.csv"),
                            "fa_fwd16_kernel")
        copy = per_dispatch(os.path.join(run_dir, f"pmc_{c}", "copy_counter_collection.csv"), "")
        copy_kib = sorted(copy.values())[-2]          # median of the three 1 GiB copies
        ideal_kib = (1 << 30) / 1024.0                # each copy reads and writes 1 GiB
        out[c] = {"kib_per_dispatch": float(np.mean(list(main.values()))), "dispatches": len(main),
                  "copy_kib": copy_kib, "scale": ideal_kib / copy_kib}
    c = CONFIGS[MAIN]
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    algorithmic = 4 * B * H * N * d * 2 + B * H * N * 4          # Q, K, V in, O out (bf16), LSE
    fetch = out["FETCH_SIZE"]["kib_per_dispatch"] * 1024 * out["FETCH_SIZE"]["scale"]
    write = out["WRITE_SIZE"]["kib_per_dispatch"] * 1024 * out["WRITE_SIZE"]["scale"]
    summary = {
        "kernel": "fa_fwd16_kernel<bf16, d=128, non-causal, bf16 out>",
        "workload": "B=8 H=16 N=2048 d=128 bf16 non-causal forward (bench.py main leg)",
        "commands": TRAFFIC_COMMANDS + [f"python3 bench.py --traffic-summary <out>"],
        "counters": out,
        "hbm_fetch_bytes_per_launch": fetch,
        "hbm_write_bytes_per_launch": write,
        "hbm_bytes_per_launch": fetch + write,
        "algorithmic_bytes_per_launch": algorithmic,
        "traffic_over_algorithmic": (fetch + write) / algorithmic,
        "code_sha256": source_hash(),
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(summary, f, indent=1)
    print(json.dumps(summary, indent=1))


TRAFFIC_COMMANDS = [
    "rocprofv3 --pmc FETCH_SIZE -d <out>/pmc_FETCH_SIZE -o main -f csv -- python3 bench.py --only-main --steps 3 --warmup 1 --no-cpu",
    "rocprofv3 --pmc FETCH_SIZE -d <out>/pmc_FETCH_SIZE -o copy -f csv -- python3 bench.py --copy-calib",
    "rocprofv3 --pmc WRITE_SIZE -d <out>/pmc_WRITE_SIZE -o main -f csv -- python3 bench.py --only-main --steps 3 --warmup 1 --no-cpu",
    "rocprofv3 --pmc WRITE_SIZE -d <out>/pmc_WRITE_SIZE -o copy -f csv -- python3 bench.py --copy-calib",
]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Leg:
    def __init__(self, name, fn, flops=0.0, bytes_=0.0):
        self.name, self.fn, self.flops, self.bytes = name, fn, flops, bytes_
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


def build_legs(dev):
    legs = []
    c = CONFIGS[MAIN]
    q, k, v = (t.to(dev) for t in make_qkv(**c))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    fl = attention_flops(B, H, N, d, False)
    legs.append(Leg("bf16_fwd_b8h16n2k_d128", lambda: fa.fwd(q, k, v, False, out=o, lse=lse), fl))
    legs.append(Leg("bf16_fwd_b8h16n2k_d128_causal",
                    lambda: fa.fwd(q, k, v, True, out=o, lse=lse), fl / 2))
    c8 = CONFIGS[FP8]
    B8, H8, N8, d8 = c8["B"], c8["H"], c8["N"], c8["d"]
    q8, k8, v8 = (t.to(dev) for t in make_qkv(**c8))
    signs = torch.from_numpy(make_signs(H8, d8, c8["seed"])).to(dev)
    pq, pk, pv = (fa.fp8_alloc_packed(B8, H8, N8, d8, dev) for _ in range(3))
    o8 = torch.empty((B8, H8, N8, d8), dtype=torch.bfloat16, device=dev)
    lse8 = torch.empty((B8, H8, N8), dtype=torch.float32, device=dev)
    nel = B8 * H8 * N8 * d8
    prep_bytes = 3 * (nel * 2 + nel + B8 * H8 * (N8 // 128) * 4)

    def prep():
        fa.fp8_prep(q8, signs, 128, out=pq)
        fa.fp8_prep(k8, signs, 128, out=pk)
        fa.fp8_prep(v8, None, 128, out=pv)

    legs.append(Leg("fp8_prep_qkv_b4h16n4k_d128", prep, 0.0, prep_bytes))
    legs.append(Leg("fp8_fwd_b4h16n4k_d128",
                    lambda: fa.fwd_fp8(pq, pk, pv, B8, H8, N8, d8, False, out=o8, lse=lse8),
                    attention_flops(B8, H8, N8, d8, False)))
    keep = (q, k, v, o, lse, q8, k8, v8, signs, pq, pk, pv, o8, lse8)
    return legs, keep


def build_next_legs(dev):
    """Legs of the rows beyond the forward; timed apart from the step."""
    legs = []
    c = CONFIGS[MAIN]
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
    c8 = CONFIGS[FP8]
    B8, H8, N8, d8 = c8["B"], c8["H"], c8["N"], c8["d"]
    q8, k8, _ = (t.to(dev) for t in make_qkv(**c8))
    signs = torch.from_numpy(make_signs(H8, d8, c8["seed"])).to(dev)
    pq, pk = (fa.fp8_alloc_packed(B8, H8, N8, d8, dev) for _ in range(2))
    nel = B8 * H8 * N8 * d8
    rope_bytes = 2 * (nel * 2 + nel + B8 * H8 * (N8 // 128) * 4)

    def prep_rope():
        fa.fp8_prep(q8, signs, 128, out=pq, rope=("half", 10000.0, 0))
        fa.fp8_prep(k8, signs, 128, out=pk, rope=("half", 10000.0, 0))

    legs.append(Leg("fp8_prep_rope_qk_b4h16n4k_d128", prep_rope, 0.0, rope_bytes))
    keep += [q8, k8, signs, pq, pk]
    # microscaled fp8: prep of Q, K (along d, Hadamard) and V (along N), then
    # the forward on the same workload
    v8 = make_qkv(**c8)[2].to(dev)
    mq, mk, mv = (torch.empty(fa.mx_packed_bytes(B8, H8, N8, d8), dtype=torch.uint8, device=dev)
                  for _ in range(3))
    mx_bytes = 3 * (nel * 2 + nel + nel // 32)

    def prep_mx():
        fa.mx_prep(q8, signs, "d", out=mq)
        fa.mx_prep(k8, signs, "d", out=mk)
        fa.mx_prep(v8, None, "n", out=mv)

    legs.append(Leg("fp8_mx_prep_qkv_b4h16n4k_d128", prep_mx, 0.0, mx_bytes))
    o8 = torch.empty((B8, H8, N8, d8), dtype=torch.bfloat16, device=dev)
    lse8 = torch.empty((B8, H8, N8), dtype=torch.float32, device=dev)
    for causal in (False, True):
        legs.append(Leg("fp8_mx_fwd_b4h16n4k_d128" + ("_causal" if causal else ""),
                        lambda causal=causal: fa.fwd_fp8(mq, mk, mv, B8, H8, N8, d8, causal, out=o8,
                                                         lse=lse8, mx=True),
                        attention_flops(B8, H8, N8, d8, causal)))
    keep += [v8, mq, mk, mv, o8, lse8]
    # block-scaled fp8, causal (the non-causal forward is in the step)
    bq, bk, bv = (fa.fp8_prep(t, sg, 128) for t, sg in ((q8, signs), (k8, signs), (v8, None)))
    legs.append(Leg("fp8_fwd_b4h16n4k_d128_causal",
                    lambda: fa.fwd_fp8(bq, bk, bv, B8, H8, N8, d8, True, out=o8, lse=lse8),
                    attention_flops(B8, H8, N8, d8, True)))
    keep += [bq, bk, bv]
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
    for _ in range(warmup):
        for L in legs:
            L.run(False)
    torch.cuda.synchronize()
    events = [[L.run(True) for L in legs] for _ in range(steps)]
    torch.cuda.synchronize()
    for step in events:
        for L, (a, b) in zip(legs, step):
            L.times.append(a.elapsed_time(b) * 1e-3)


def leg_summary(L):
    t = float(np.mean(L.times))
    e = {"ms": t * 1e3, "ms_min": float(np.min(L.times)) * 1e3}
    if L.flops:
        peak = PEAK_FP8 if L.name.startswith("fp8") else PEAK_BF16
        e["tflops"] = L.flops / t / 1e12
        e["frac_of_peak"] = e["tflops"] / peak
    if L.bytes:
        e["gbps"] = L.bytes / t / 1e9
        e["frac_of_hbm"] = e["gbps"] / PEAK_HBM
    return e


def cpu_baseline():
    """The float64 oracle on one step of the timed workload (about 15 s on
    16 host cores), on the same seeded inputs: the bf16 forward, non-causal
    and causal, B=8 H=16 N=2048 d=128 (the oracle computes every score and
    masks; the metric counts half for causal), and the fp8 leg as the
    fake-quant oracle (random-sign Hadamard + per-128-row e4m3 quantisation of
    the outlier inputs, then exact attention) at B=4 H=16 N=4096 d=128.
    Value: the step's metric flops over the oracle's time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    c, c8 = CONFIGS[MAIN], CONFIGS[FP8]
    b, b8 = c["B"], c8["B"]
    q, k, v = (t[:b].to(torch.float64).numpy() for t in make_qkv(**c))
    q8, k8, v8 = (t[:b8].to(torch.float64).numpy() for t in make_qkv(**c8))
    signs = make_signs(c8["H"], c8["d"], c8["seed"])
    fl = (attention_flops(b, c["H"], c["N"], c["d"], False)
          + attention_flops(b, c["H"], c["N"], c["d"], True)
          + attention_flops(b8, c8["H"], c8["N"], c8["d"], False))
    t0 = time.perf_counter()
    oracle.attention(q, k, v, False)
    oracle.attention(q, k, v, True)
    oracle.fake_quant_attention(q8, k8, v8, signs, 128, False)
    el = time.perf_counter() - t0
    return {"value": fl / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"one step: bf16 B={b} H=16 N=2048 d=128 non-causal and causal; fp8 fake-quant "
                      f"(Hadamard + block e4m3) B={b8} H=16 N=4096 d=128 outlier inputs; float64 numpy "
                      f"oracle, {el:.1f} s"}


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
    ap.add_argument("--only-main", action="store_true",
                    help="only launch the bf16 non-causal forward (for counter runs)")
    ap.add_argument("--source-hash", action="store_true", help="print the kernel source hash")
    ap.add_argument("--traffic-summary", metavar="DIR",
                    help="write the HBM-traffic summary from the counter runs under DIR (no GPU)")
    args = ap.parse_args()
    if args.source_hash:
        print(source_hash())
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
    legs, _keep = build_legs(dev)
    if args.only_main:
        legs = legs[:1]
    for _ in range(args.warmup):
        for L in legs:
            L.run(False)
    torch.cuda.synchronize()
    log(f"warmup done; timing {args.steps} steps")
    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        events.append([L.run(True) for L in legs])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for step in events:
        for L, (a, b) in zip(legs, step):
            L.times.append(a.elapsed_time(b) * 1e-3)
    total_flops = sum(L.flops for L in legs)
    step_s = wall / args.steps
    legs_out = {L.name: leg_summary(L) for L in legs}
    dom = legs[0]
    t_dom = float(np.mean(dom.times))
    achieved = dom.flops / t_dom / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16, "traffic": measured_traffic(),
            "kernel": "fa_fwd16_kernel<bf16,128,noncausal>", "launch_ms": t_dom * 1e3}
    out = {
        "metric": "attention fwd TFLOP/s (4*B*H*N^2*d, /2 causal), bf16 and fp8",
        "value": total_flops / step_s / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp8",
        "data": "synthetic",
        "config": {"workload": "bf16 fwd B=8 H=16 N=2048 d=128 (non-causal + causal) + fp8 "
                               "prep/fwd B=4 H=16 N=4096 d=128 (0.1% outliers)",
                   "global_batch": 8, "seq_len": 2048, "head_dim": 128, "heads": 16,
                   "parallelism": "single-gpu"},
        "legs": legs_out,
        "roofline": roof,
    }
    if not args.only_main and not args.no_next:
        log("timing the rows beyond the forward")
        nlegs, _nkeep = build_next_legs(dev)
        time_legs(nlegs, args.steps, args.warmup)
        out["next_rows"] = {L.name: leg_summary(L) for L in nlegs}
    if not args.no_cpu:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
