"""CPU fp64 oracle for the sparse-MQA decode path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The GPU library
never does, and this package imports nothing from the GPU library: the two
share no code.  Inputs come from ``synth`` (random draws and storage
encoders only).

What it computes (sources: the vLLM blog post "DeepSeek-V4.1-Flash sur vLLM :
5x de débit agentique dès le jour 0" and the CocoLoop news digest of it):

* ``ref.score``   — indexer scoring ("logits MQA creux", blog §Kernels): for a
  query t and every position j it may see, S[t,j] = sum_h w[t,h] *
  max(0, kappa_j * <qI[t,h], kI[j]>).  Dense mode scores every position
  0..p_t; candidate mode scores only a given candidate list (the late indexer
  layers' fixed 16K-candidate set).
* ``ref.topk``    — top-k position selection (the DeepSelect step, blog
  §TL;DR and §Kernels): the k best positions by (score desc, position asc).
* ``ref.attend``  — sparse MQA attention (MegaAttention, blog §Kernels) over
  the selected FP4 global-latent rows plus the FP8 sliding-window rows of the
  last 128 positions (blog §"SWA bounded replay"; digest §"Les particularités
  du modèle lui-même"), one softmax over the union, window clipped at the
  replay start s (blog §"Côté encodeur").
* ``ref.attend_fp8kv`` — the same attention over an FP8 global cache (E4M3
  rows times a row scale), the format the FP4 cache replaced (digest §"Les
  particularités du modèle lui-même": the FP4 cache is about 45% smaller).
* ``ref.attend_nvfp4`` — the same attention over a global cache in the NVFP4
  layout the pages name (E2M1, an E4M3 scale per 16 elements, an fp32 tensor
  scale).
* ``ref.attend_fused`` — MegaAttention's fused form (blog §Kernels): query
  RoPE, the attention, inverse RoPE on the output and FP8 conversion.
* ``ref.decode_step`` — the three in sequence.
* ``brute`` — the same definitions as pure-Python loops for tiny inputs.

Every function evaluates its definition directly, in float64, on values
decoded exactly from the stored bytes (``codecs``).  Readings taken where the
pages are silent are listed in the design doc of the repository and restated at
each function.

Parity status: codecs, score, topk, attend, attend_fp8kv and attend_nvfp4 are pinned by closed forms,
brute force, textbook special cases and invariants (tests/test_oracle.py,
tests/test_codecs.py, tests/golden/).  Two readings cannot be pinned against
any number printed on the pages — the ReLU-weighted indexer form and K = V
(the shared latent row serves as key and value) — and are marked
"parity unpinned" against the pages in ``ref``.
"""
from . import codecs, ref, brute  # noqa: F401
