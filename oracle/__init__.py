"""CPU oracle for the quantized-LoRA hot path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. It shares no code with the HIP library (no kernels, headers,
tables or constant generators) and never imports it.

It is written to be checked by eye against the pages it follows:

* QLoRA page -- Heng's Blog, "QLoRA: Efficient Finetuning of Quantized LLMs"
  (heng-blog.pages.dev/blog/qlora): the layer equation in the introduction,
  NF4 in section "贡献一：4-bit NormalFloat（NF4）" (Contribution 1) and double
  quantization in section "贡献二：Double Quantization" (Contribution 2).
* LowRA page -- the cloud.tencent.com.cn write-up of LowRA: per-output-channel
  quantization with custom thresholds (section 3, workflow), groups of 64
  scaled by absmax (section 4.1), mappings and thresholds (section 4.1,
  figure 3) and the weighted Lloyd-Max learner (section 5).
* LowRA page, sections 3 and 5: the LoftQ-style low-rank initialiser (five
  alternating quantize / rank-r SVD steps).
* AQLoRA page -- bittide.aicompass.dev translation of AQLoRA, section 3.1
  (profiling pass): the per-layer NF4 round-trip error.
* LoRAQuant page -- "LoRAQuant: Mixed-Precision Quantization of LoRA to
  Ultra-Low Bits", method overview and key design: SVD reparameterization of
  the adapter and mixed-precision quantization of its components.

Floating point follows IEEE binary32/binary64 with round to nearest even and
subnormals kept. numpy's float32 operators are single correctly rounded
operations, so ``np.float32(a) / np.float32(b)`` is the IEEE quotient.

Functions without an independent pin say "parity unpinned" in their
docstring; at present there are none.
"""

from . import bf16, fp8, nf4, dq, layer, codebook, lloyd, loftq, loraquant, sizes  # noqa: F401
