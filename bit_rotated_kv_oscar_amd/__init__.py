"""MI355X (gfx950) library for OSCAR's INT2 KV-cache write and mixed-precision
paged decode attention.  The work runs in liboscar.so (HIP); this package is
its thin binding.  Importing it loads the library and fails if it is missing.
"""
from ._lib import OscarError, load
from .api import (BF16_PAGES_PER_REQ, HEAD_DIM, N_RECENT, N_SINK, PAGE, LayerCache, Rotation,
                  bf16_decode_workspace_bytes, bf16_paged_decode, calib_accumulate, calib_accumulate_heads,
                  calib_rotations, calibrate_per_head, calibrate_rotation, clip_threshold,
                  decode_attn, decode_attn_noalloc, decode_step, decode_workspace_bytes, extend_attn,
                  hist_block_bytes, profile_events, read_probe, rotation_bytes, write_kv)

load()
