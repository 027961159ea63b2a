"""CPU oracle for the selective state-space scan: TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct float64 NumPy statement of
what the scan and the single-token state update compute. It exists so that
the HIP kernels can be checked against something written independently of
them. Only the test suite, the package's smoke check and the benchmark's CPU
baseline leg may import it. The product path never calls it, and it shares
no code, tables or helpers with the HIP library or its Python binding.

Sources, cited by tag throughout:

- [HiddenCost]  kongchang.com, "Mamba的隐藏代价：逃离二次内存却难逃二次参数需求"
                (the hidden cost of Mamba).
- [TtoM]        ybb.press, "从 Transformer 到 Mamba：状态空间模型如何重塑序列计算的效率边界"
                (from Transformer to Mamba).
- [Paradigm]    intelliparadigm.com, "Mamba架构：突破Transformer瓶颈的序列建模新范式".
- [Breakthrough] ruibaoantu.com, "Mamba新突破：SSM架构挑战注意力机制，引领推理新范式".
- [Notes]       lyirs.cc, "Mamba" (study notes on Gu & Dao 2023).
"""

from .conv_oracle import causal_conv1d, causal_conv1d_update  # noqa: F401
from .scan_bwd_oracle import selective_scan_bwd  # noqa: F401
from .ssd_oracle import ssd_quadratic, ssd_recurrent  # noqa: F401
from .ssm_oracle import (  # noqa: F401
    softplus,
    silu,
    discretize_delta,
    input_coefficient,
    selective_scan,
    selective_state_update,
    scaled_error,
)
