"""Oracle for the 2-bit routed-expert MoE layer: a plain, slow, CPU-only
reference written from the definition (NumPy, fp64 after decoding).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg may import, call or run anything in this package.
It shares no code with the HIP library (bit_quantized_routed_amd); the only
code both sides use is the seeded input generator package `synth`.

    q2.decode_blocks / encode_blocks   the Q2 super-block codec
    q4.decode_blocks / encode_blocks   its 4-bit sibling
    moe.q8_rows                        Q8 activations of the routed experts
    moe.route / bucket / ffn / layer   the MoE layer
    moe.rmsnorm_bf16 / stack           the residual stack with RMSNorm
"""
from . import q2, q4, moe  # noqa: F401
