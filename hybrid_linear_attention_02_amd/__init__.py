"""MI355X-native GDN recurrent-state update: slot pool, decode, chunked prefill.

The compute path is the HIP library ``libgdn.so`` (built from ``csrc/``); the
``gdn`` module is a thin ctypes binding over its C ABI. ``workloads`` draws the
seeded synthetic inputs.
"""
