"""Compressed-KV GQA decode path for AMD MI355X (gfx950): hand-written HIP kernels behind a C ABI
(include/kvc.h), with a thin ctypes binding. Importing the package loads nothing; the HIP library is loaded on
first use and every entry point fails loudly if it has not been built."""

__all__ = ["abi", "configs", "synth", "session"]
