"""Float64 CPU oracle for decode attention over a rank-compressed KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
path (``rank_compressed_kv_kvlr_amd``) and imports nothing from it.

What it computes (all in float64, plain numpy, no blocking or fusion):

* storage of keys and values as latents, K_lat = K P_K and V_lat = V P_V
  (StiefAttention technical summary, "Metodologia: StiefAttention" >
  "Mecanismo Central", item 5 "Inferência"; the German page "Don't be so
  Stief!", "Technisches Resümee" > "Kernmechanismus" > "Inferenz"; the pages
  print the key side only, the value side is read by symmetry);
* reconstruction K~ = K_lat P_K^T, V~ = V_lat P_V^T before standard softmax
  attention (same passages), one basis pair per KV head with its own ranks
  (STAR-KV technical summary, "Metodologia" section 1, "Inferenza": hard
  thresholds truncate the projections per decoder block and attention head);
* the same quantity in latent order, q~ = q P_K, scores K_lat q~, and
  (p V_lat) P_V^T, which is equal by associativity;
* the folded form, where the bases sit in the caller's query and output
  projections: q~ in, o_lat = p V_lat out (StiefAttention, "Mecanismo
  Central" item 5; STAR-KV, "Metodologia" section 2).

* mixed-precision latent storage (``oracle/quant.py``): block-wise Hadamard
  folded into the bases, 4-bit outlier and 3-bit inlier blocks per token,
  and decode over the dequantised latents (STAR-KV technical summary,
  "Metodologia" section 3), pinned in tests/test_quant_oracle.py.

* joint values with per-head keys (``oracle/joint.py``): the values of all
  heads of a token share one latent V_all P_J, and head h reconstructs with
  its own rows of P_J (STAR-KV technical summary, "Metodologia" section 2),
  pinned in tests/test_joint_oracle.py.

Pins (tests/test_oracle_pins.py): orthonormality of the bases, the textbook
softmax attention at full rank, invariance under P -> P O, definition mode
equals latent mode, a 50-digit mpmath brute force on tiny shapes, closed
forms (T=1, q=0, T=2, values inside span(P_V)), the folded output against
the brute force through o_lat = o P_V, hand-derived golden
examples under tests/golden/, and a planted-mistake battery showing that a
dropped term, a wrong scale, a swapped basis, a wrong head mapping or an
off-by-one length each fails at least one pin. No function here is
"parity unpinned".
"""
from .kvlr_oracle import (  # noqa: F401
    bf16_round,
    compress,
    reconstruct,
    softmax,
    attend,
    attend_reconstructed,
    attend_latent,
    decode,
    decode_latents,
    attend_folded,
    decode_folded,
    decode_head_reconstructed,
    decode_head_latent,
    kv_head_of,
)
from . import joint, quant  # noqa: F401
