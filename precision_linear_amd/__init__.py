"""MI355X-native FP8 (e4m3fn) scaled matrix multiply.

The compute runs in the HIP library `libfp8_scaled_mm.so` (built from
`csrc/`); `fp8_scaled_mm` below only marshals torch tensors into the C ABI.
The library is loaded on first use and its absence is an error.
"""
PER_TENSOR = 0
ROWWISE = 1


def __getattr__(name):
    if name in ("fp8_scaled_mm", "lib", "Fp8MMError", "status_string", "config_names",
                "select_config", "library_path"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
