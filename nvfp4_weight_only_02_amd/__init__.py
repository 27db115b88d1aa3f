"""MI355X-native NVFP4 weight-only projection GEMV for batched LLM decode.

The compute lives in a HIP library (``csrc/``) behind a C ABI
(``include/nvfp4.h``); this package only marshals torch tensors into it.  The
library is loaded on first use; every entry point raises if it is missing.
"""
