"""MI355X-native TTT-E2E prefill: a C-ABI HIP library and its Python binding.

Importing the package does not load the HIP library; `binding.load()` does,
and raises if the built library is missing.
"""
__all__ = ["synth", "binding"]
