"""OCTOPUS KV-cache codec and the attention that reads it, on MI355X (gfx950).

The compute path is liboctopus.so (C ABI in include/octopus.h, HIP kernels in
csrc/); binding.py is its thin Python binding.  workloads.py holds the seeded
synthetic inputs.  The codebook artifact under codebooks/ is an input to the
codec (Lloyd-Max tables, Sec. 3.4 of the OCTOPUS paper).
"""
from .binding import (Codec, OctoError, PackedCache, lib, octo_attend_chunk,  # noqa: F401
                      octo_attend_decode, octo_attend_decode_noalloc,
                      octo_chunk_workspace_bytes, octo_decode_step,
                      octo_decode_tokens,
                      octo_decode_step_workspace_bytes, octo_decode_workspace_bytes, octo_encode,
                      octo_record_sizes, workspace)
