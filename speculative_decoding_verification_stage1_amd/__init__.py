"""MI355X-native fused LLM sampling and speculative verification.

The compute path is the HIP library ``libss.so`` (C ABI in ``include/ss.h``);
``_lib`` is its thin ctypes binding and ``workloads`` holds the seeded input
generators.  Import ``speculative_decoding_verification_stage1_amd._lib``
to use the library; it raises if the library has not been built.
"""
__all__ = ["workloads"]
