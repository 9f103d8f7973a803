"""Seeded synthetic RAG workloads shared by the tests, the oracle checks and the
benchmark. Holds no attention, RoPE or metadata-packing arithmetic: it only
draws documents (Zipf), places them at logical positions, and fills tensors
with seeded N(0, 1) values rounded to bf16."""
from .rag import (  # noqa: F401
    CONFIGS, CONFIG_ORDER, Config, Group, Workload, RequestLayout, Segment, build, make,
    layouts_for, zipf_ranks, f32_to_bf16_bits, BF16_NAN, harmonic,
)
