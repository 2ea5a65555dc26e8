"""MI355X-native selective state-space causal scan (prefill + decode) for one GPU's channel slice.

``prefill`` and ``decode_step`` call the C ABI of include/ssm.h (libssm.so, hand-written
HIP kernels for gfx950) through a thin ctypes binding; ``q8_quantize`` and
``q8_dequant_sum`` call the block int8 codec of include/ssm_codec.h; ``Projector``,
``conv_silu`` and ``conv_xproj`` call the channel-sliced projections, the conv front and the two
fused, of include/ssm_proj.h; ``decode_fused`` runs a decoded token's conv front, x_proj, dt_proj and
decode step in two kernels (include/ssm_layer.h); ``inputs`` makes seeded synthetic workloads.  Importing the
package does not load the library; the first call does, and raises if it is not built.
"""
from ._lib import (PROJ_DT, PROJ_IN, PROJ_OUT, PROJ_X, Projector, SsmError, conv_silu, conv_xproj,  # noqa: F401
                   decode_fused, decode_fused_workspace_bytes, decode_step, decode_step_pool, load, prefill,
                   prefill_pool, q8_dequant_sum, q8_num_blocks, q8_quantize, workspace_bytes)
