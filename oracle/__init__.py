"""CPU oracle for hierarchical hash retrieval decode and the HISA indexer variant.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the graft entry
point's smoke check and the benchmark's CPU-baseline leg may import anything
here.  The oracle shares no code with the HIP path (no kernels, headers,
helpers, tables or constant generators); the only thing both sides consume is
the seeded input generator, which holds none of the method's arithmetic.

Everything is plain numpy in fp64 on the exact stored input values (bf16 or
f32 keys/values, f32 queries and projections, fp8 e4m3fn index keys).

Sources (page titles as printed):
  [HHR]  "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation"
         (arXiv 2610.01230) -- abstract, Figures 1-4, appendix Tables 3-4.
  [HATA] "HATA: Trainable and Hardware-Efficient Hash-Aware Top-k Attention
         for Scalable Large Model Inference" (arXiv 2506.02572) -- abstract.
  [HISA] "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse
         Attention" (arXiv 2603.28458) -- abstract.
"""
from . import hhr, hisa  # noqa: F401
