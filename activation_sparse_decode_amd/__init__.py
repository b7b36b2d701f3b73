"""MI355X-native activation-sparse FFN / projection decode.

The compute path lives in the HIP library ``libsparse_ffn.so`` (C ABI,
``include/sparse_ffn.h``); ``binding`` marshals torch tensors into it.
``synth`` holds the seeded synthetic inputs.  Importing the package loads
nothing; ``binding`` loads the library on first use.
"""
