"""MI355X-native Kimi Delta Attention (KDA) forward: chunked prefill and
recurrent decode behind a C-ABI HIP library (libkda.so).

Importing the package loads nothing; the library is loaded on first use by
``gated_delta_rule_04_amd.kda`` and the call fails loudly if it is missing.
"""

__version__ = "0.1.0"
