"""MI355X-native gated delta rule: forward and VJP behind the libgdr C ABI.

The kernels are hand-written HIP for gfx950 (csrc/); ``binding`` marshals
torch tensors to the C entry points declared in include/gdr.h.
"""

from .binding import (GdrError, SavedChunks, gdr_backward, gdr_backward_workspace, gdr_calib_copy,
                      gdr_calib_mfma, gdr_forward, gdr_forward_noalloc, gdr_forward_workspace, gdr_keeps_chunks,
                      gdr_profile_enable, gdr_profile_read, lib)

__all__ = ["GdrError", "SavedChunks", "gdr_forward", "gdr_forward_noalloc", "gdr_backward", "gdr_forward_workspace",
           "gdr_backward_workspace", "gdr_keeps_chunks", "gdr_profile_enable", "gdr_profile_read",
           "gdr_calib_copy", "gdr_calib_mfma", "lib"]
