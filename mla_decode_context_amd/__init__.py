"""MI355X-native absorbed-MLA decode with decode context parallelism (DCP).

The computation lives in libmla.so (hand-written HIP for gfx950 behind the C ABI
of include/mla.h).  ``binding`` marshals torch tensors into that ABI, ``runner``
drives one DCP decode step (every rank's partial, then the merge) on one GPU,
and ``workloads`` builds seeded synthetic inputs.  Importing the package does
not load the library; the first call does, and fails loudly if it is missing.
"""
from .binding import (MlaError, load_library, mla_dcp_local_seqlens, mla_decode_partial,
                      mla_lse_merge, mla_merge_v_up_proj, workspace_size)

__all__ = ["MlaError", "load_library", "mla_dcp_local_seqlens", "mla_decode_partial",
           "mla_lse_merge", "mla_merge_v_up_proj", "workspace_size"]
