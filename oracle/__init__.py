"""CPU oracle for the MLA decode step -- TEST INFRASTRUCTURE, not the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The HIP library
never routes through it, and this package imports nothing from the HIP
package (``head_latent_attention_11_amd``): the two share only the seeded
input generator in ``mla_inputs``, which holds no arithmetic of the method.

What it computes (plain, slow, obviously correct, float64 throughout):

* ``formats``: decoding of the stored number formats (bfloat16 bit patterns,
  OCP FP8 E4M3 codes via a 256-entry table built from the format's
  definition) and the per-token E4M3 quantisation rule of the fp8 cache.
* ``rope``: rotary position embedding, interleaved pairs.
* ``mla``: the decode step written the *naive* way that "DeepSeek-V2:
  Strong, Economical, Efficient" (Appendix C) describes before it introduces
  absorption: per head, keys k_{j,i} = [W^UK_i c_j ; k^R_j] and values
  v_{j,i} = W^UV_i c_j are materialised from the cached latent rows, then
  ordinary softmax attention with scale 1/sqrt(d_h + d_h^R) is taken
  ("DeepSeek-V3 Technical Report" notes, MLA section, attention-output
  equation).  Nothing is absorbed, blocked or fused.

Pins (tests marked "not gpu"): brute force on tiny inputs, the L = 1 and
uniform-softmax closed forms, a hand-derived worked example under
``tests/golden/``, the absorbed/un-absorbed associativity identity, library
scaled-dot-product attention, torch's float8_e4m3fn casts, RoPE's
relative-position property and the cache-size statements of the pages.
The RoPE pairing convention itself is parity unpinned (a convention the pages
cite but do not define).
"""
from . import formats, rope, mla  # noqa: F401
