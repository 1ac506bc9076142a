"""CPU oracle for the W4A16 group-quantised linear layer.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it. The HIP library never calls it.
"""
from .awq_oracle import *  # noqa: F401,F403
from .awq_oracle import (device_layout_doc, device_words, pack_canonical,  # noqa: F401
                         unpack_canonical, pack_zeros, unpack_zeros, pack_device,
                         unpack_device, dequant64, dequant16, linear64,
                         l1_scale, normalised_error, linear_bruteforce, round_output16,
                         weight_set_bytes, model_bytes, low_nibble,
                         quantize_rtn, RTN_QMAX, silu64, linear_silu_mul64,
                         silu_mul_scale)
from .attention_oracle import (ROPE_STYLES, rope_inv_freq64, rope_pairs, rope64,  # noqa: F401,E402
                               split_qkv, softmax64, decode_step64, decode_error_scale,
                               decode_bytes)
from .w4a8_oracle import (FP8_MAX, fp8_e4m3_value, fp8_e4m3_encode, quantize_act_fp8,  # noqa: F401,E402
                          linear_w4a8_64, w4a8_l1_scale)
