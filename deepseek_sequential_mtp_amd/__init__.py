"""MI355X (gfx950) implementation of the teacher-forced sequential MTP depth
chain, its shared-head masked cross-entropy (forward and backward) and draft
verification.

The compute path is the HIP library ``libmtp.so`` (C ABI in ``include/mtp.h``);
``deepseek_sequential_mtp_amd._lib`` is its ctypes binding.  ``synth`` holds the
seeded synthetic-input generators.  Importing this package does not load the
library; the binding loads it on first use and raises if it is missing.
"""


def __getattr__(name):
    if name in ("chain_forward", "head_ce_fwd_bwd", "verify", "load", "MtpError"):
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
