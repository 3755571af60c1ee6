"""Score-centering (SC) correction for AMD MI355X (gfx950).

The compute lives in ``libsc.so`` (HIP kernels behind the C ABI declared in
``include/sc.h``); ``off_policy_logit_amd.sc`` is its ctypes binding and
``off_policy_logit_amd.build`` compiles it.  Importing this package does not
load the library; the first call into ``sc`` does, and fails loudly when the
library has not been built.
"""
__all__ = ["sc", "build"]
