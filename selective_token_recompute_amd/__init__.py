"""MI355X (gfx950) engine for one denoising iteration of a masked diffusion LM
with converged-token locking (SureLock), behind the C ABI in include/dlm.h.

``engine`` holds the C-ABI calls under their own names and a small Engine
class; ``ops`` exposes the single-stage calls of include/dlm_ops.h.  Importing
this package does not load the library; the first call does, and fails loudly
if it has not been built (``python -m selective_token_recompute_amd.build``).
"""
from ._lib import LIB_PATH, DlmError, lib  # noqa: F401
