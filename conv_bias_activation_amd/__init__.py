"""MI355X (gfx950) fused contraction + bias + activation.

Thin Python binding over the C ABI of ``libbiasact.so`` (include/biasact.h):
argument marshalling only.  Every step of the computation runs in the HIP
kernels of the library; PyTorch is used here only to hand over device
pointers and the current HIP stream.  If the library is not built, importing
this package raises ImportError — there is no fallback path.

    gemm_bias_act(A, B, bias, C, act="leaky_relu", alpha=0.001)
    conv2d_bias_act(x, w, bias, y, strides=(1, 1), pads=(0, 0, 0, 0), dilations=(1, 1), act="tanh")
    gemm_bias_act_2k(..., workspace=ws) / conv2d_bias_act_2k(..., workspace=ws)
"""
from ._binding import (  # noqa: F401
    ACT_CODES,
    DTYPE_CODES,
    BiasActError,
    conv2d_bias_act,
    conv2d_bias_act_2k,
    conv2d_bias_act_workspace_size,
    conv_out_hw,
    dtypes_code,
    force_halo_variant,
    last_tile_config,
    force_tile_config,
    gemm_bias_act,
    gemm_bias_act_auto,
    conv2d_bias_act_auto,
    gemm_path,
    gemm_static_path,
    set_gemm_path,
    set_conv_path,
    conv_path,
    tune_gemm,
    tune_conv,
    gemm_bias_add_act,
    gemm_bias_add_act_2k,
    conv2d_bias_add_act,
    conv2d_bias_add_act_2k,
    gemm_bias_act_2k,
    gemm_bias_act_2k_noalloc,
    gemm_bias_act_workspace_size,
    gemm_tile_config,
    conv_tile_config,
    lib,
    lib_path,
    num_tile_configs,
    status_string,
    tile_config_name,
)
