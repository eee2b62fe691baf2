"""CPU oracle for the weight-only-quantized SwiGLU MLP.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or constant with the HIP library in ``weight_quantized_mlp_amd/`` and imports
nothing from it.

Everything is plain NumPy in float64 (the pages fix no wider precision), with
the materialisation roundings the pages prescribe (float32 dequantised FP8 and
NVFP4 weights, float16 points of the AWQ routed-expert step).  Each function
cites the page and section it follows:

* "issue: tp>1 fp8w tail-MLP shard host-dequantizes every layer", sections
  "Mechanism on the tp>1 path", "Proposed fix", "Logic anchor" -- FP8 E4M3
  per-output-channel decode and the SwiGLU MLP equation.
* "Qwen3.8-27B-NVFP4", sections "Checkpoint specification", "NVFP4 numerics
  as implemented" -- the three-level NVFP4 tensor and the 36-byte record.
* "[Kernel][SM70] Add native-g32 AWQ QPN M1 operator", section "What it
  does" -- the AWQ int4 group-32 routed-expert single-token step.
* "Qwen3.8-27B-NVFP4", section "Implemented execution path" -- the per-token
  8-bit activation quantization of the W4A8 variant (actquant.py).

Pins (what ties each function to something other than itself) are in
``tests/test_oracle.py``.  The pages print no values for the full-size MLP at
the 27B tail-layer shape; there the oracle's act and out are checked on sampled
rows against pure-Python sums over independently decoded weights.
"""
from .codecs import e4m3_to_f64, e2m1_to_f64, bf16_bits_to_f64, f16_bits_to_f64
from .dequant import (fp8w_dequant, nvfp4_dequant, nvfp4_dequant_parts, awq_dequant, awq_dequant_parts,
                      awq_dequant_bias, awq_bias_bits)
from .pack import (block64_pack, block64_unpack, awq_bank_layout, awq_pack_bank,
                   awq_unpack_bank)
from .mlp import silu, swiglu_mlp, mlp_fp8w_ref, mlp_nvfp4_ref, mlp_nvfp4_w4a8_ref, mlp_bruteforce
from .actquant import token_exponent, e4m3_encode_rne, quant_e4m3_per_token
from .moe import moe_awq_m1_ref, moe_w13_stage_ref, moe_w2_stage_ref, moe_bruteforce
from .metric import normwise_rel_err

__all__ = [n for n in dir() if not n.startswith("_")]
