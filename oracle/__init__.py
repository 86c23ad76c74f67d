"""CPU oracle for the QMoE routed expert FFN — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy code that states what the operator computes.  Only
the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import it; the product path never does.  It shares no code with the HIP
library.

Parity pins (see tests/test_oracle.py): every function here is checked
against values fixed by the pages or by mathematics.  One reading stays
unpinned by the pages (nibble order inside a packed byte); it is pinned only
as a stated convention.
"""
from .qmoe_oracle import (  # noqa: F401
    ContractError, validate, route, expert_permutation, dequantize, activation,
    qmoe, qmoe_dense, qmoe_tokens, expert_ffn, local_experts,
)
from .grouped_matmul import grouped_matmul, grouped_matmul_rows  # noqa: F401
from .moe_oracle import moe, moe_tokens, moe_validate, moe_activation, gelu  # noqa: F401
