"""MI355X-native GPT-2 decoder forward: a HIP C-ABI library (libgpt2.so) and its ctypes binding.

Importing the package loads nothing; the library is opened on first use by
``decoder_only_transformer_gpt2_amd.gpt2``.
"""
