"""CPU oracle for the KIVI-style quantized KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never imports it and this package never imports the
library: the two share no code, headers, tables or helpers.  The only shared
module is ``kvq_synth`` (seeded input draws, no method arithmetic).

What it computes, and from where:

* ``codec``     -- the quantizer, restore and the two quantization axes of the
  "KV Cache Quantization Strategies" exercise (page 1, Step 2 table and the
  Step 4 reference solution: ``_quantize``, ``restore``,
  ``quantize_key_per_channel``, ``quantize_value_per_token``).  Arithmetic in
  float32, as the page's ``x.float() * scale``; round half to even.
* ``cache``     -- ``append_and_partition``: residual window, overflow-only
  flush, append-only segments, token counters (page 1, Step 3 and Step 4
  TODO 3), generalised to whole-group flushes.
* ``attention`` -- softmax(sigma q k^T) v with causal visibility and the GQA
  head mapping, in float64, straight from its definition ("KV Cache and
  autoregressive video generation", section 3.1 equations and the section 04
  ``attn_full`` / ``attn_step`` description).
* ``layout``    -- the library's packed byte layout, written out from its
  specification (the pages do not fix a packing; see the docstring there).
* ``ledger``    -- byte budgets ("KV Cache quantization and compression",
  sections 01 and 05; page 1 ``compare``).
* ``axis_study`` -- asymmetric-axis against same-axis grouped quantization
  (page 1, Step 2 table and section 5.1), measured on the synthetic
  workloads; the block-attention frame mask lives in ``attention``
  ("KV Cache and autoregressive video generation", section 6.3).

Parity status of every function is stated in its module header.
"""
from . import codec, cache, attention, layout, ledger  # noqa: F401
from .codec import (quantize_with_scale, scale_from_absmax, quantize_key_per_channel,
                    quantize_value_per_token, restore)  # noqa: F401
from .cache import KVQuantizationStrategies  # noqa: F401
