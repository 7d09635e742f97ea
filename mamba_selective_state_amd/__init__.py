"""Mamba-2 selective state update (SSU) decode for AMD MI355X (gfx950).

The update runs in hand-written HIP kernels behind a C ABI (include/ssu.h,
libssu.so); this package is its Python binding.
"""
from .ssu import (LIBRARY_PATH, SsuArgs, SsuConvShiftArgs, SsuError, SsuReplayArgs, SsuReplayLpArgs,
                  SsuSsdArgs, mx8_quantize, replay_lp_selective_state_update,
                  ssu_mx8_quantize, ssu_replay_lp_update, make_replay_lp_args,
                  mx4_quantize, replay_mx4_selective_state_update, ssu_mx4_quantize,
                  ssu_replay_mx4_update,
                  batch_memcpy, ssd_combined_fwd_varlen, ssu_ssd_prefill, ssu_ssd_workspace_bytes,
                  ssu_ssd_prefill_noalloc, make_ssd_args, SSD_SCRATCH_BYTES, ssu_ssd_plan,
                  prewarm_ssd_combined_fwd_varlen, SsuSsdPlanDesc,
                  conv_state_shift, make_args, make_conv_shift_args, make_replay_args,
                  prewarm_selective_state_update, replay_selective_state_update,
                  replay_spec_selective_state_update, selective_state_update, ssu_abi_version,
                  ssu_batch_memcpy, ssu_conv_state_shift, ssu_last_error, ssu_plan,
                  ssu_replay_spec_update, ssu_replay_update, ssu_update)

__all__ = ["selective_state_update", "prewarm_selective_state_update",
           "replay_selective_state_update", "replay_spec_selective_state_update", "ssu_update",
           "ssu_replay_update", "ssu_replay_spec_update", "ssu_plan", "ssu_last_error",
           "ssu_abi_version", "make_args", "make_replay_args", "SsuArgs", "SsuReplayArgs",
           "SsuError", "LIBRARY_PATH", "batch_memcpy", "conv_state_shift", "ssu_batch_memcpy",
           "ssu_conv_state_shift", "make_conv_shift_args", "SsuConvShiftArgs",
           "ssd_combined_fwd_varlen", "ssu_ssd_prefill", "ssu_ssd_workspace_bytes", "SsuSsdArgs",
           "ssu_ssd_prefill_noalloc", "make_ssd_args", "SSD_SCRATCH_BYTES", "ssu_ssd_plan",
           "prewarm_ssd_combined_fwd_varlen", "SsuSsdPlanDesc",
           "replay_lp_selective_state_update", "ssu_replay_lp_update", "make_replay_lp_args",
           "SsuReplayLpArgs", "mx8_quantize", "ssu_mx8_quantize", "mx4_quantize",
           "replay_mx4_selective_state_update", "ssu_mx4_quantize", "ssu_replay_mx4_update"]
