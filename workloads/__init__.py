"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays out the *inputs* of the path:
context lengths, block tables, query and cache contents, the new token's K/V.
It holds none of the method's arithmetic (no slot mapping, no cache layout, no
softmax). Both the CPU oracle tests and the HIP path consume what it returns.

Recipes follow the workloads the pages describe:
  * paging in fixed 16-token blocks reached through a per-sequence block table
    ("Anthropic Interview: Design an LLM Inference API with GPU Batching",
    Key concepts / Paged KV memory; "MLSys Engineer - Inference Systems Q&A", Q1);
  * prompts of about 1,500 tokens with up to 300 generated, some reaching
    100,000 tokens (same interview page, opening problem statement);
  * a shared system-prompt prefix held once in the pool
    ("Forward Deployed Engineering Interview", Ch.2 section 8, paging and
    prefix caching).

All values are N(0,1) drawn in float32 and, for bf16 workloads, rounded to bf16
by round-to-nearest-even on the bit pattern. Arrays that hold bf16 data are
returned as uint16 bit patterns, float32 data as uint32 bit patterns, so every
consumer sees identical bits.
"""
from .configs import (  # noqa: F401
    Workload,
    DecodeStep,
    make_workload,
    CONFIG_NAMES,
    f32_to_bf16_bits,
    bits_dtype,
)
