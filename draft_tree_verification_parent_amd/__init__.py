"""MI355X (gfx950) implementation of one round of tree speculative decoding.

The compute lives in libgraft.so (HIP kernels behind the C ABI declared in
include/graft.h); `api` is its Python binding and `verify_round` drives one
round through it on a single HIP stream.
"""
from ._native import GraftError, LIB_PATH  # noqa: F401
