"""MI355X-native sparse ternary BitLinear (Sparse-BitNet / BitNet b1.58 forward and backward).

The compute path lives in ``libbitlinear.so`` (hand-written HIP for gfx950, C ABI declared in
``include/bitlinear.h``); ``sparsity_amd.bitlinear`` is a thin ctypes binding with the same
names.  PyTorch is used only to own device memory and streams.
"""
from .bitlinear import (  # noqa: F401
    BL_BWD_ACCUM_DW, BL_BWD_ACCUM_DX, BL_DTYPE_BF16, BL_DTYPE_F32, BL_LAYOUT_DENSE2,
    BL_LAYOUT_SPARSE, BitLinearError, BlBwdDesc, BlBwdGroupPlan, BlFwdDesc, BlFwdXDesc, BlPackDesc,
    BlGemmGroupPlan, BlPackGroupPlan, BlQuantDesc, act_quant_group, act_quant_i8_group, BwdGroup, FusedGroup, FwdGroup, GemmGroup, PackGroup,
    act_quant, act_quant_i8, bitlinear_gemm_group, bitlinear_gemm_group_build,
    bitlinear_gemm_group_plan,
    bitlinear_bwd, bitlinear_bwd_group, bitlinear_pack_group, bitlinear_pack_group_build,
    bitlinear_pack_group_plan,
    bitlinear_bwd_group_build, bitlinear_bwd_group_plan, bitlinear_bwd_workspace_bytes,
    bitlinear_fwd, bitlinear_fwd_group, bitlinear_fwd_group_fused, bitlinear_group_build,
    bitlinear_group_fused_build, bitlinear_group_fused_table_bytes, bitlinear_group_table_bytes,
    bitlinear_pack, bitlinear_packed_bytes, bwd, bwd_workspace_bytes, fwd, lib, pack,
    packed_bytes, bitlinear_pack_noalloc, BlChainLayer, BlChainPlan, Chain, bitlinear_chain_plan,
    bitlinear_chain_build, bitlinear_fwd_chain, BL_LAYOUT_SPARSE6, bitlinear_transcode6,
    transcode6,
)
