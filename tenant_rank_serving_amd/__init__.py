"""Delta-CoMe mixed-precision delta apply for AMD Instinct MI355X (gfx950).

The compute lives in libdeltacome.so (C ABI, include/deltacome.h): hand-written
HIP kernels for gfx950 plus a host packer.  This package is its thin Python
binding; torch supplies device memory and streams only.
"""
from ._lib import (  # noqa: F401
    DC_ERR_ALIGN, DC_ERR_BUFFER, DC_ERR_HIP, DC_ERR_INVALID_ARG, DC_ERR_RANGE, DC_ERR_SHAPE,
    DC_ERR_UNSUPPORTED, DC_MAX_GROUP, DC_MAX_TENANTS, DC_OK, DC_SCRATCH_BYTES, DC_OP_DECODE, DC_OP_MULTITENANT, DC_OP_PREFILL,
    EXPORTS, LIB_PATH, MultitenantCall, REGIONS, DcError, DeltaView, dc_algorithmic_bytes, dc_apply_decode,
    dc_apply_multitenant, dc_apply_multitenant_group, dc_apply_multitenant_noalloc, dc_apply_multitenant_timed, dc_apply_prefill, STAGES, dc_check_spec, dc_dequant, dc_pack, dc_pack_codes,
    dc_allocate_bits, dc_pack_device, dc_packed_bytes, dc_region, dc_status_string, dc_unpack, dc_workspace_bytes, dc_group_workspace_bytes, GroupCall, lib, make_spec,
    DC_KIND_BITDELTA, DC_KIND_LOWRANK, BaselineGroupCall, BaselineView, dc_apply_baseline_multitenant,
    dc_apply_baseline_multitenant_group, dc_baseline_algorithmic_bytes, dc_baseline_bytes,
    dc_baseline_workspace_bytes, dc_pack_bitdelta, dc_pack_lowrank,
    DC_ERR_MAX_WIDTHS, dc_error_table, dc_error_table_workspace_bytes, dc_svd, dc_svd_workspace_bytes,
)
