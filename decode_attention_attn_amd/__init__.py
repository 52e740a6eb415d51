"""MI355X-native MFA decode attention (libmfa) and its Python binding.

``decode_attention_attn_amd.mfa`` loads the HIP library ``libmfa.so`` built
from ``csrc/`` and exposes its C entry points with the same names.
``decode_attention_attn_amd.inputs`` draws the seeded synthetic inputs.
Importing the package itself loads nothing.
"""
