"""MI355X-native fused scaled-dot-product attention: tiled prefill FMHA on
bf16 MFMA, paged split-KV decode with a log-sum-exp merge, and shared-prefix
cascade decode, as hand-written HIP for gfx950 behind the C ABI declared in
``include/attn.h``.

Importing the package loads nothing; the HIP library is loaded on the first
call into :mod:`attention_tiled_fmha_amd.attn`.
"""
__all__ = ["attn", "workloads"]
