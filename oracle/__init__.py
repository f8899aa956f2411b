"""CPU oracle for the HyQuant decode path. TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy code (float64 unless a step fixes a
narrower precision) that states what the HIP library must compute. Only the
tests, the smoke check and the CPU-baseline leg of the benchmark may import
it; the library and its Python binding never do, and this package imports
nothing from them.

Sources, cited by page and section (no page prints a worked example):
  [AFS] "HyQuant ... Explained for Beginners", aifromscratch.in:
        "How It Works: The Hybrid-Precision Strategy" (three token sets,
        window of the last 128 tokens, 4-bit keys and values) and
        "The Technical Mechanics" (prefill overlay; decode dequantizes on
        the fly inside attention).
  [WPN] "Hybrid-precision attention reduces compute cost ...", wpnews.pro,
        body paragraph 4 (detector: accumulate queries, one matmul every
        64 tokens, column sums).
  [KQ]  kipquest.com paper page, "The abstract".
  [HP]  hotpaper.ai paper page, technical-approach list (vertical-line
        tokens from column-wise attention scores, under 5 %).

Where the pages are silent the readings are those listed in the design notes
(quantizer format: asymmetric min-max INT4, 32-channel groups along head_dim,
fp16 scale and fp16 zero point = group minimum; one softmax over all three
token sets; raw-logit column scores; lower index wins score ties).

Modules: ``quant`` (INT4 encode/decode), ``attention`` (hybrid decode
attention and the LSE merge), ``detect`` (vertical-line detector),
``prefill`` (hybrid prefill operator), ``lifecycle`` (the rolling cache over
many decode steps: re-detection every R steps among the positions that still
have 16-bit rows).
"""
from . import quant, attention, detect, prefill, lifecycle  # noqa: F401
