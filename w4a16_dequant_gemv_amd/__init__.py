"""W4A16 group-wise INT4 weight quantization and fused-dequant GEMV/GEMM for
AMD Instinct MI355X (gfx950).

The arithmetic runs in the HIP library `libw4a16.so` behind a C ABI
(`include/w4a16.h`, and `include/kv_codec.h` for the KV-cache codec in
`w4a16_dequant_gemv_amd.kv`, and `include/w8a8.h` for W8A8 with SmoothQuant in
`w4a16_dequant_gemv_amd.w8a8`, `include/producers.h` for GPTQ and AWQ in
`w4a16_dequant_gemv_amd.producers`); this package only marshals torch tensors into it.
Submodules load lazily so that the seeded input generators in `synthetic`
can be imported on machines without the library.
"""
import importlib

__all__ = ["quantize_pack", "dequant", "gemv", "gemm", "linear", "kernel_config", "QuantizedWeight",
           "W4A16Error", "synthetic", "kv", "w8a8", "producers"]


def __getattr__(name):
    if name in ("quantize_pack", "dequant", "gemv", "gemm", "linear", "kernel_config",
                "QuantizedWeight", "W4A16Error"):
        api = importlib.import_module(".api", __name__)
        return getattr(api, name)
    if name in ("synthetic", "kv", "w8a8", "producers"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
