"""CPU oracle for the Beam MoE block -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and nothing here
imports the product path.
"""
from .beam_moe_oracle import *  # noqa: F401,F403
from .fp8_weights import *  # noqa: F401,F403
from .beam_attention_oracle import *  # noqa: F401,F403
from .beam_dense_oracle import *  # noqa: F401,F403
