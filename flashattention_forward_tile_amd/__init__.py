"""MI355X-native FlashAttention-2 forward pass (gfx950, HIP).

Importing the package loads nothing; ``fa2`` loads the compiled C-ABI library
on first use and fails loudly if it has not been built.
"""
__all__ = ["workloads"]
