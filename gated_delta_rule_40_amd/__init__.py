"""MI355X-native Kimi Delta Attention (KDA) recurrence.

The compute lives in ``libkda.so`` (hand-written HIP for gfx950 behind a C
ABI, declared in ``include/kda.h``); ``gated_delta_rule_40_amd.libkda`` is the
thin ctypes binding over it and ``gated_delta_rule_40_amd.inputs`` draws the
seeded synthetic inputs.  Importing this package loads nothing.
"""
