"""CPU oracle for the chunk-wise causal attention path — TEST INFRASTRUCTURE.

Plain, slow, obviously correct numpy code that states what the hot path
computes.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it; the library and its Python binding never do, and nothing
here imports them.  The two sides share only the seeded input generator,
which holds none of the method's arithmetic.

Sources:
  [WF]  "Wave Forcing: Towards Speed-of-Light Streaming Video Generation"
        §3.1 (chunk-wise causal mask, context order), §4.2 (K/V published
        after QKV projection and RoPE into paged attention slots).
  [SD2] "Interpretation: The AI-Generated Future" (StreamDiffusionV2),
        "Adaptive sink and RoPE refresh": RoPE phases are a caller policy,
        so positions are explicit inputs.

Modules:
  numerics   bfloat16 <-> float32 storage conversions (round-to-nearest-even)
  rope       3D rotary embedding (double-precision angles, float rotation)
  publish    paged scatter of K/V into the pool through the page table
  attention  masked softmax attention per query slot, float64
  brute      the same attention with explicit per-key loops (tiny inputs)
  history    end-of-round history rotation as a page-table reordering
  mx         MXFP8 (E4M3 + E8M0 block scale) keys and queries for the
             8-bit QK^T variant, and its attention
  qkv        QKV projection (one float64 product, one rounding) followed
             by the publish: what the fused projection epilogue must produce

Parity status: every function here is pinned by tests/test_oracle_*.py
against closed forms, textbook/library special cases, invariants the pages
fix, and brute force.  The pages print no numeric example for attention or
RoPE, so no pin uses the pages' own numbers for them.
"""
