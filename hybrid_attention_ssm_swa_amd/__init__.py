"""MI355X (gfx950) implementation of the Hymba hybrid-head mixer.

The computation lives in libhymba_mixer.so (HIP kernels + hipBLASLt GEMMs
behind a C ABI, include/hymba_mixer.h).  This package is its Python binding:
``_lib`` mirrors the C functions by name; ``layer.MixerLayer`` manages device
memory (torch) around one layer, ``griffin.GriffinBlock`` around one Griffin
recurrent block.  Importing works without the library; the
first call loads it and raises if it has not been built.
"""
from ._lib import (  # noqa: F401
    HYMBA_BF16, HYMBA_F16, HYMBA_F32, HymbaError, LIB_PATH, EXPORTED, load_library,
    hymba_layer_cfg, hymba_layer_weights, hymba_kv,
    hymba_layer_persistent_bytes, hymba_layer_create, hymba_layer_destroy, hymba_kv_share_bind,
    hymba_mixer_workspace_bytes, hymba_layer_prepare, hymba_mixer_prefill, hymba_mixer_decode,
    hymba_layer_meta_outputs, hymba_last_error, hymba_status_string,
    hymba_kernel_attention, hymba_kernel_selective_scan, hymba_kernel_epilogue, hymba_kernel_gemm_rows,
    hymba_kernel_gemm_rows_workspace,
    hymba_kernel_selective_scan_workspace,
    hymba_layer_profile, hymba_layer_profile_read, hymba_stage_name, HYMBA_N_STAGES,
    hymba_layer_check, hymba_layer_set_overlap, HYMBA_ERR_RANGE, HYMBA_ERR_UNSUPPORTED,
    hymba_mixer_decode_static, HYMBA_ERR_INVALID_ARG, HYMBA_ERR_WORKSPACE,
    griffin_block_cfg, griffin_block_weights, griffin_block_persistent_bytes, griffin_block_prepare,
    griffin_workspace_bytes, griffin_block_prefill, griffin_block_decode, GRIFFIN_N_STAGES,
)
