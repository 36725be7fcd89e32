"""MI355X-native HBM slot buffer for dynamic sparse attention decode over a
host-offloaded KV cache: hash matching, sort-free eviction (lifetime or
bucketed LRU), miss-only gather from pinned host memory and split-k decode
attention, as HIP kernels for gfx950 behind the C ABI of include/avsg.h."""
from . import avsg  # noqa: F401

__all__ = ["avsg"]
