"""attention_state_memory_amd: attention-state memory (ASM) on MI355X.

The compute runs in the HIP library ``libasm_amd.so`` (C ABI declared in
``include/asm_memory.h``); the functions exported here marshal torch device
tensors into that ABI.  Importing the package does not load the library;
the first call does, and raises if it is missing.
"""
__all__ = ["api", "synth"]
