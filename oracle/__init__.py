"""CPU oracle for the QLoRA NF4 linear layer -- test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the GPU library never does.
"""
from .qlora_oracle import *  # noqa: F401,F403
from .qlora_oracle import (nf4_levels_f64, nf4_levels_f32, uniform4_levels_f32, fp4_levels_f32,  # noqa: F401
                           quantize_codes, nf4_quantize, pack_nibbles, unpack_nibbles,
                           blockwise_absmax, e4m3_value, e4m3_encode, round_rational_to_f32,
                           exact_sum_f32, mean_f32, double_quant, dequant_constants,
                           bf16_round, bf16_to_f64, dequant_weight, lora_scale, linear_fwd, linear_fwd_f64, linear_bwd_f64,
                           linear_bwd, storage_bits_per_param, quantize_layer,
                           quantize_layer_bf16, bf16_round_f64, merge_weight, e2m1_value)
