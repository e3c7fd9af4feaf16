"""Hybrid compressed attention (CSA + HCA) of DeepSeek-V4 for AMD MI355X (gfx950).

The compute lives in libhcsa.so (hand-written HIP kernels behind the C ABI declared in
include/hcsa.h); `long_context_attention_26_amd.hcsa` is its ctypes binding.
"""
__all__ = ["hcsa"]
