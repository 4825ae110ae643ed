"""MI355X (gfx950) RAWINT4 routed-expert MoE LoRA layer: forward and backward.

The compute lives in ``libkt_rawint4.so`` (hand-written HIP kernels behind the C
ABI of ``include/kt_rawint4.h``); this package only binds it (``_lib``) and
provides seeded synthetic workloads (``workloads``).
"""

from ._lib import (  # noqa: F401
    KT_RAWINT4_EHIP,
    KT_RAWINT4_EINVAL,
    KT_RAWINT4_EWORKSPACE,
    KT_RAWINT4_FORMAT_MXFP4,
    KT_RAWINT4_FORMAT_RAWINT4,
    KT_RAWINT4_OK,
    LIBRARY_PATH,
    KtRawInt4Error,
    kt_rawint4_dequant,
    kt_rawint4_dequant_mxfp4,
    kt_rawint4_group,
    kt_rawint4_group_workspace_bytes,
    kt_rawint4_last_error,
    kt_rawint4_moe_bwd,
    kt_rawint4_moe_bwd_recompute,
    kt_rawint4_moe_diagnostics,
    kt_rawint4_moe_fwd,
    kt_rawint4_moe_infer,
    kt_rawint4_moe_infer_workspace_bytes,
    kt_rawint4_moe_layer,
    kt_rawint4_moe_workspace_bytes,
    kt_rawint4_profile_enable,
    kt_rawint4_profile_phase_name,
    kt_rawint4_profile_read,
    kt_rawint4_unpack,
    kt_rawint4_weight_layout,
    load_library,
    make_layer,
)
