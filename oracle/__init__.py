"""fp64 CPU oracle of the GPTQ hot path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use it.
"""
from .gptq_oracle import *  # noqa: F401,F403
from .gptq_oracle import (GRID_ASYM, GRID_TERNARY, QuantResult, boundary_distance, damp,
                          fit_grid, gptq_quantize, hessian, hessian_factor, inverse_hessian_factor,
                          layer_loss, layer_loss_tokens, maxq_of, pack_codes,
                          quantize_layer, rtn_quantize, unpack_codes)
