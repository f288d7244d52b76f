"""CPU oracle for the fused FP8 x FP4 top-k MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library.

It is a plain, slow, obviously correct numpy implementation of what the layer
computes, following the pages' description step by step:

  codecs   E4M3 / E2M1 / E8M0 formats and the power-of-two block quantiser
  moe_ref  routing, counting-sort bucketisation, activation quantisation,
           grouped GEMM1 + SwiGLU*weight epilogue, grouped GEMM2, combine
  blockfp8 the block-FP8 (128 x 128 weight blocks, float32 scales) variant of
           the expert MLP, on moe_ref's routing, bucketisation and combine

Sources (web pages, cited by title and section):
  [MegaMoE notes]  "MegaMoE" study notes (obnotes), sections "Dispatch阶段",
                   "Expert矩阵权重量化", "GEMM", "WorkSpace", "L1 epilogue",
                   "原始权重布局", "L2 epilogue".
  [MegaMoE fusion] "MegaMoE：把通信和计算融合到一个 Mega Kernel", sections
                   "核心实现机制", "Python API 调用流程".
  [Warp spec]      "Warp Specialization: DeepEP vs Mega MoE", epilogue and
                   combine excerpts.
  [Counting sort]  "05.10 Counting Sort / Bucketization 在 DeepGEMM Mega MoE 中的映射",
                   sections 2.1-2.3, 5.2, 7.1, 9.1.
  [MonoMoe]        "MonoMoe kernel — design", the fixed-shape paragraph (block-FP8
                   128 x 128 weights) and §1 (five-phase pipeline).

Parity status: every function here is pinned by tests under tests/ against
format definitions, torch casts, brute force and invariants, except the
end-to-end value of y at the large shapes, for which the pages print no worked
example (it is pinned only through those component pins).
"""
