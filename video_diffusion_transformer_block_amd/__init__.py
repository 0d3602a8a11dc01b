"""MI355X (gfx950) implementation of the Wan2.1 DiT denoising step.

The computation lives in ``libwandit.so`` (hand-written HIP kernels behind the
C ABI of ``include/wan_dit.h``); :mod:`.binding` marshals torch device tensors
into that ABI.  Build the library with ``python -m
video_diffusion_transformer_block_amd.build`` (or ``__graft_entry__.build()``).
"""
from . import binding  # noqa: F401
from .binding import (NOALLOC_SCRATCH_BYTES, Cfg, WanError, attention_fwd, attention_8bit_fwd, attention_8bit_q_fwd,  # noqa: F401
                      attention_8bit_quantize, attention_8bit_workspace_bytes, block_fp8_bytes,
                      block_fp8_workspace_bytes,
                      block_weights, dit_block_fp8_fwd, dit_block_fwd, dit_block_fwd_noalloc, dit_block_noalloc_bytes, quantize_block_fp8,
                      model_fp8_bytes, fp8_workspace_bytes, quantize_model_fp8, dit_step_fp8_fwd,
                      sample_fp8_fwd,
                      dit_step_cached_fwd, dit_step_fwd, euler_fwd, i2v_mask, kv_cache_bytes,
                      kv_cache_fwd, lib, linear_fp8_fwd, linear_fwd, ln_modulate_fwd, make_cfg, model_weights, sample_fwd,
                      quantize_rows_fp8, quantize_tensor_fp8, sample_workspace_bytes, set_attention_events, status_str,
                      tmlp_fwd, tmlp_weights, workspace_bytes)
