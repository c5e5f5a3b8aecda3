"""MI355X-native Lynx progressive KV-cache quantization.

The compute path is the HIP library ``liblynx.so`` (sources in ``csrc/``,
C ABI in ``include/lynx.h``); ``long_context_serving_amd.lynx`` is its thin
Python binding.  Importing this package loads nothing; import
``long_context_serving_amd.lynx`` to load the library.
"""
__all__ = ["lynx", "synth"]
