"""Reference oracle for the low-bit KV cache — TEST INFRASTRUCTURE ONLY.

A plain, slow, CPU implementation of what the GPU path computes, written
directly from the formulas of the pages it cites. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path (the HIP library and its Python binding) never
imports, calls or falls back to anything here, and this package imports
nothing from the product path; the two share only the seeded input
generators, which hold none of the method's arithmetic.

Sources (by page title and section):
  [P2-int]  "KV Cache Quantization — 8-bit and 4-bit", section
            "Integer quantization in one screen": the affine quantizer, its
            scale and zero-point, the int8/int4 ranges and the scale/2 bound.
  [P2-size] same page, "The bytes-per-token formula" and "A worked memory
            example".
  [P2-gran] same page, "Granularity: per-tensor, per-token, per-channel",
            "The outlier problem: keys have outlier channels" and "Why keys and
            values want different treatment".
  [P2-dec]  same page, "Decode is memory-bound, so smaller is also faster".
  [P1-kivi] "Sub-8-Bit KV Cache Quantization Is Not a Free Lever for an RDNA4
            Agent Swarm", FAQ and "What the low-bit numbers actually cost"
            (per-channel keys, per-token values, fp residual, KVQuant's
            dense-and-sparse outliers); "Why 8 bits hides the problem and 4 bits
            exposes it" (2 bits = four levels).
  [P3-fmt]  "KV Cache Quantization Benchmarked: 8-bit Is Nearly Lossless, How
            Much Does 4-bit Cost?", the memory paragraph of "KV Cache
            Quantization: 8-bit Is Essentially Free" (8-bit caches at about
            32-34 KiB per token against 64 KiB) and the glossary paragraph
            (fp8_e4m3: 4-bit exponent, 3-bit mantissa; q8_0 / q4_0: blocks
            of 32 elements sharing a scale).

Modules:
  quant   group quantize / dequantize (affine and symmetric), integer ranges,
          dense-and-sparse split
  fp8     fp8 E4M3 elements: decoding from the bit layout, rounding encode
  cache   the cache state machine (append, residual flush; affine, fp8 and
          symmetric 32-element block formats), the documented
          packed byte layout, dequantized tensors, float64 attention, and the
          log-sum-exp merge of split partials (softmax_partial, merge_partials)
  sizes   the bytes-per-token formula and the actual cache sizes
  rope    the rotary embedding applied to pre-RoPE cached keys inside
          attention (KVQuant's pre-RoPE keys, [P1-kivi]); textbook RoPE, since
          the pages define none: parity unpinned by the pages, pinned by the
          embedding's own properties

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, invariants and brute force. One part has no pin in
the pages: the bit layout of the packed bytes (``cache.pack``), which is this
library's own documented format; its pin is the unpack/pack identity only
("parity unpinned" by the pages). The split merge is not on the pages either;
it is pinned by its closed form (merged partials of any split equal the
unsplit softmax result).
"""
