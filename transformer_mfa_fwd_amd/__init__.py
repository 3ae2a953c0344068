"""transformer_mfa_fwd_amd -- fused attention forward (libmfa) for MI355X.

``fwd(q, k, v, ...)`` runs the HIP library through its C ABI (include/mfa.h);
see ``_binding.fwd`` for the arguments.  ``decode_len`` is the decode over a
device-held cache length (``_binding.decode_len``; ``decode_len_noalloc`` the
same with its scratch in static device memory), ``decode_masked`` the
single-query decode over a cache whose valid keys a device mask marks, ``packed_qkv_fwd`` the
bidirectional forward over sequences packed in one fused QKV tensor, and
``varlen_fwd`` the forward over separate query and key packings, ``bwd`` the
gradients of the forward.  The package holds the HIP sources
(csrc/), their build step (build.py), the ctypes binding and the seeded input
generators (workloads.py).
"""
from ._binding import (  # noqa: F401
    EXPORTED, LIB_PATH, MFAError, PATH_AUTO, PATH_GENERIC, PATH_MFMA, PATH_NAMES,
    PATH_SPLIT_DECODE, bwd, bwd_workspace_size, decode_len, decode_len_noalloc, decode_len_workspace_size, decode_masked,
    decode_masked_workspace_size, fwd, load_library, packed_qkv_fwd, plan, set_kernel_events,
    varlen_fwd, varlen_workspace_size, version, workspace_size,
)
