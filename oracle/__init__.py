"""Plain CPU oracle for the fused exact-attention forward pass.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything in this package. The
GPU library never calls it, and it shares no code, table or constant with the
HIP kernels: both sides are written independently from the pages.

Everything here is slow, obviously correct numpy in float64 unless a function
says otherwise. Sources, cited by page title and section:

* "FlashAttention - one, two, three!" (Medium), section "Standard Attention":
  the materialised S = QK^T, softmax, PV computation that the fused kernel must
  reproduce exactly.
* same page, sections "FlashAttention v1." and "FlashAttention v2.": the
  online softmax with a separately tracked denominator and the deferred
  normalisation (the formulas themselves are missing from the text).
* "FlashAttention-3: Fast & Accurate Attention with Asynchrony &
  Low-Precision" (Embodied AI 101 transcript), section "Incoherent Processing
  for FP8 Accuracy": random-sign Hadamard rotation of Q and K before FP8
  quantisation, fused into the rotary-embedding step; and the review "FlashAttention-3: почему внимание стало
  быстрее", section "Метод", item 3: block quantisation.

Modules:
    attention   naive materialised-softmax attention (the definition)
    online      blockwise online-softmax emulator (pins the recurrence)
    hadamard    fast Walsh-Hadamard transform with random signs
    fp8         OCP e4m3 ("fn") rounding / encoding from the format definition
    quant       block / per-tensor fp8 quantisation and fake-quant attention
    backward    gradients dQ, dK, dV of exact attention (chain rule, materialised)
    rope        rotary position embedding (interleaved or half pairing)
    mx          microscaled e4m3 quantisation (power-of-two scale per 32 elements)
    decode      the same attention for few query rows over a long, ragged key
                history (grouped key/value heads, bottom-right causal)

Parity pins for every function live in tests/test_oracle_*.py. Functions whose
result has no independent pin are marked "parity unpinned" in their docstring.
"""

from .attention import attention, attention_rows, softmax_probs  # noqa: F401
from .online import attention_online  # noqa: F401
from .hadamard import fwht, random_sign_hadamard  # noqa: F401
from .fp8 import e4m3_round, e4m3_encode, e4m3_decode, E4M3_MAX  # noqa: F401
from .quant import fp8_quantize, fp8_dequantize, fake_quant_attention, pow2_ceil_f32  # noqa: F401
from .backward import attention_backward, attention_delta  # noqa: F401
from .decode import attention_decode, visible_keys  # noqa: F401
from .rope import rope, rope_angles, rope_cos_sin, rope_frequencies  # noqa: F401
from .mx import mx_quantize, mx_dequantize, fake_quant_attention_mx  # noqa: F401
