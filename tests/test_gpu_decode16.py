"""GPU parity of the decode-shaped forward (fa_fwd_decode through the C ABI)
against the float64 decode oracle on the same seeded, 16-bit-rounded inputs.

Every output element is compared (the oracle is cheap for few query rows),
with the forward's tolerances: max-abs <= 4e-3 and RMSE <= 5e-4 on O with
float32 output (beyond half an ulp with 16-bit output), LSE within 1e-3.
Rows that see no key must come out as O = 0, LSE = -inf exactly. The cases
cover grouped heads, several row groups, ragged and empty sequences, causal
rows with fewer keys than queries, more splits than key blocks, one split
(no merge), all three head dims and both input types; the two decode
workloads run at full size in the configuration the benchmark times.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import exact_attention_55_amd as fa
from exact_attention_55_amd.inputs import DECODE_CONFIGS, make_decode, to_f64

from helpers import check_lse, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_case(B, H, Hkv, Nq, Nk, d, causal, dtype, lens, splits, out_f32, seed=21, scale=None):
    q, k, v, _ = make_decode(B, H, Hkv, Nq, Nk, d, seed, dtype)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32)
    return compare(q, k, v, sl, causal, dtype, splits, out_f32, scale)


def compare(q, k, v, sl, causal, dtype, splits, out_f32, scale=None, where=""):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    sld = None if sl is None else sl.to(DEV)
    o, lse = fa.fwd_decode(qd, kd, vd, causal=causal, softmax_scale=scale, seqlens_k=sld,
                           num_splits=splits, out_f32=out_f32)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    lens = None if sl is None else sl.numpy().tolist()
    o_ref, lse_ref = oracle.attention_decode(to_f64(q), to_f64(k), to_f64(v), causal, scale, lens)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"rows without keys differ {where}"
    assert np.all(o[empty] == 0.0), f"rows without keys must be zero {where}"
    live = ~empty
    if np.any(live):
        check_o(o[live], o_ref[live], "f32" if out_f32 else dtype, where)
        check_lse(lse[live], lse_ref[live], where)
    return int(np.sum(empty))


SMALL = [
    # B, H, Hkv, Nq, Nk, d, causal, dtype, seqlens, splits
    (2, 4, 4, 1, 1000, 128, False, "bf16", None, 1),
    (2, 4, 4, 1, 1000, 128, False, "bf16", None, 4),
    (2, 8, 2, 1, 777, 128, True, "bf16", [777, 300], 0),
    (3, 8, 1, 4, 513, 64, True, "fp16", [513, 5, 0], 3),
    (1, 32, 4, 5, 2000, 128, True, "bf16", None, 7),          # 40 rows: two row groups
    (2, 2, 2, 3, 65, 256, True, "bf16", [65, 2], 2),          # L = 2 < Nq = 3
    (1, 1, 1, 1, 1, 64, False, "bf16", None, 1),
    (1, 16, 16, 1, 4096, 64, False, "fp16", None, 0),
    (1, 2, 2, 1, 40, 128, False, "bf16", None, 16),           # more splits than blocks
    (2, 6, 3, 2, 3000, 256, False, "fp16", [3000, 1234], 5),
    (1, 4, 2, 33, 700, 128, True, "bf16", [690], 3),          # 66 rows, causal tail
    (4, 8, 8, 1, 257, 128, True, "bf16", [0, 0, 0, 0], 2),    # every sequence empty
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,dtype,lens,splits", SMALL)
@pytest.mark.parametrize("out_f32", [True, False])
def test_small_full_compare(B, H, Hkv, Nq, Nk, d, causal, dtype, lens, splits, out_f32):
    where = f"B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} {dtype} lens={lens} splits={splits} f32={out_f32}"
    say("decode " + where)
    run_case(B, H, Hkv, Nq, Nk, d, causal, dtype, lens, splits, out_f32)


def test_non_default_scale_and_split_invariance():
    """Scale 0.3; the result does not depend on the number of splits beyond
    rounding (1, 2, 5 and 64 splits all meet the oracle bound)."""
    for s in (1, 2, 5, 64):
        say(f"decode scale 0.3 splits {s}")
        run_case(2, 8, 4, 2, 3333, 128, True, "bf16", [3333, 2500], s, True, scale=0.3)


def test_few_keys_bf16():
    """Sequences of two or three keys (one part each, so the exact split of
    P is taken), 64 sequences x 16 heads, bf16, every element with float32
    O; and the same sequences under 4 splits (parts of 0 .. 1 keys)."""
    lens = [2, 3] * 32
    for splits in (1, 4):
        say(f"decode few keys splits {splits}")
        run_case(64, 16, 16, 1, 64, 128, False, "bf16", lens, splits, True, seed=23)


@pytest.mark.parametrize("name", sorted(DECODE_CONFIGS))
def test_full_workload(name):
    """The benchmark's decode workloads, full size, in its launch
    configuration (the suggested split count), every element compared."""
    c = DECODE_CONFIGS[name]
    say(f"decode full {name}")
    q, k, v, sl = make_decode(**c)
    compare(q, k, v, sl, c["causal"], c["dtype"], 0, False, where=name)
