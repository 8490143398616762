"""Fused scaled dot-product attention forward for MI355X (gfx950).

``softmax(scale * Q K^T [+ causal mask]) V`` with MHA / GQA / MQA head
grouping, computed by hand-written HIP kernels behind the C ABI declared in
``include/attn.h`` (library ``libattn.so``). The Python binding in
:mod:`scaled_dot_product_09_amd.attn` only marshals arguments.
"""

__all__ = ["attn", "workload"]
