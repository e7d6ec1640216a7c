"""CPU oracle for sparse MLA attention over a paged latent cache -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may import this
package. The product path (the HIP library and its binding) never calls it.
"""

from .sfa_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    f32_to_bf16_bits_rne,
    dequant_int8_chain,
    resolve_rows,
    gather_latents,
    sparse_mla_attention,
    sparse_mla_attention_token,
    allclose_report,
)
