"""MI355X-native causal kernelized linear attention (gfx950 HIP + C ABI)."""
