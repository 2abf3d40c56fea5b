"""Build libfa.so in-tree with hipcc for gfx950.

    python -m exact_attention_55_amd.build [-v]
    python -m exact_attention_55_amd.build --variant NAME -DMACRO=VALUE ...

The second form builds a variant of the library with the given macros (the
kernels' compile-time switches: FA16_PINGPONG, FA16_PRIO, FA16_SCHED,
FA16_CFG_128, ...) into exact_attention_55_amd/variants/libfa_NAME.so, for
ablations: setting FA_LIB to that path makes the binding load it instead.

Each translation unit under csrc/ is compiled in parallel, then linked into
exact_attention_55_amd/libfa.so. Flags:
  --offload-arch=gfx950                  the only target
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                         no packed fp32 VALU instructions
  -fhip-fp32-correctly-rounded-divide-sqrt
                                         IEEE float32 division (the fp8
                                         quantiser's x / scale)
"""

import concurrent.futures
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfa.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["fa_api.hip", "fa_fwd16.hip", "fa_fwd16_pipe.hip", "fa_fwd_fp8.hip", "fa_fp8_prep.hip",
           "fa_bwd16.hip", "fa_decode16.hip"]
# Per-source flags. fa_fwd16_pipe.hip and fa_bwd16.hip: the compiler's MFMA
# builtins write vector registers (score tiles feed the exponentials
# directly), while the long-lived accumulators (O of the pipelined forward,
# the gradients at d = 256) stay in the accumulation registers through asm.
EXTRA_FLAGS = {"fa_fwd16_pipe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "fa_bwd16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(src, verbose, defines=(), objdir=BUILD):
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA_FLAGS.get(src, []) + list(defines) + [
        "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    usage = _resource_usage(r.stderr)
    with open(os.path.join(objdir, os.path.splitext(src)[0] + ".resources.txt"), "w") as f:
        for name, u in usage.items():
            f.write(f"{name} {u}\n")
    spilled = {n: u for n, u in usage.items()
               if u.get("ScratchSize [bytes/lane]", 0) > _scratch_allowance(n)}
    if spilled:
        raise RuntimeError(f"kernels of {src} use scratch (register spills or stack):\n  " +
                           "\n  ".join(f"{n}: {u}" for n, u in spilled.items()))
    if verbose:
        other = "\n".join(l for l in r.stderr.splitlines() if "kernel-resource-usage" not in l)
        if other.strip():
            print(other, flush=True)
    return obj


# Kernels allowed a little scratch, with the reason (bytes per lane):
#  * the one-wave-per-SIMD 16-bit forward at d = 256 (512 registers, all in
#    use): a long-lived value or two saved in the prologue and reloaded in the
#    epilogue, outside the key loop.
SCRATCH_ALLOWANCE = [
    (re.compile(r"^_ZN2fa15fa_fwd16_kernelIDF16[b_]Li256E"), 32),
]


def _scratch_allowance(name):
    for pat, limit in SCRATCH_ALLOWANCE:
        if pat.match(name):
            return limit
    return 0


def _resource_usage(stderr):
    """Per-kernel register and scratch figures from the compiler's
    kernel-resource-usage remarks. A kernel that needs scratch (spilled
    registers) is refused: every spill sits in the key loop's data path."""
    usage, cur = {}, None
    for line in stderr.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass", 1)[0].strip()
        key, _, val = body.partition(":")
        key, val = key.strip(), val.strip()
        if key == "Function Name":
            cur = val
            usage[cur] = {}
        elif cur is not None and val.lstrip("-").isdigit():
            usage[cur][key] = int(val)
    return usage


def build(verbose=False, variant=None, defines=()):
    """Compile and link the library; with variant, the ablation build of that
    name with the given -D flags (see the module docstring)."""
    objdir, out = BUILD, OUT
    if variant is not None:
        if not re.fullmatch(r"[A-Za-z0-9_]+", variant):
            raise ValueError(f"variant name {variant!r}: letters, digits and _ only")
        objdir = os.path.join(BUILD, "variant_" + variant)
        out = os.path.join(HERE, "variants", f"libfa_{variant}.so")
        os.makedirs(os.path.dirname(out), exist_ok=True)
    os.makedirs(objdir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, objdir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    _check_undefined(tmp)
    os.replace(tmp, out)
    return out


def _check_undefined(lib):
    """A shared library links even when a kernel's host launch stub was never
    emitted (the host pass drops it silently when it cannot compile
    something in the kernel's device code); such a library only fails when
    it is loaded. Refuse any undefined symbol of the library's own namespace."""
    r = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}:\n{r.stderr}")
    own = [l.split()[-1] for l in r.stdout.splitlines() if l.split() and l.split()[-1].startswith("_ZN2fa")]
    if own:
        raise RuntimeError("undefined symbols of namespace fa in the built library:\n  " + "\n  ".join(own))


if __name__ == "__main__":
    args = sys.argv[1:]
    name = None
    if "--variant" in args:
        name = args[args.index("--variant") + 1]
    defs = [a for a in args if a.startswith("-D")]
    print(build(verbose="-v" in args, variant=name, defines=defs))
