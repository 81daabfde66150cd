"""Fused attention-input epilogue (bias + NeoX rotary + KV-cache store) for MI355X.

The compute path is the HIP library ``libqkv_epilogue.so`` (C ABI in
``include/qkv_epilogue.h``); ``qkv_bias_rope_amd.binding`` is its ctypes front
end and loads the library on import (it raises if the library is not built:
there is no fallback).  ``qkv_bias_rope_amd.workloads`` holds the seeded
synthetic input generators.
"""
import importlib

__all__ = ["binding", "workloads", "Epilogue"]


def __getattr__(name):
    if name == "Epilogue":
        return importlib.import_module(".binding", __name__).Epilogue
    raise AttributeError(name)
