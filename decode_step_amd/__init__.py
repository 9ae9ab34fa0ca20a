"""MI355X-native Qwen2-style GQA decode step: libqd.so (HIP kernels for gfx950
behind the C ABI in include/qd.h) and its thin ctypes binding."""
from . import qd
from .qd import QdError

__all__ = ["qd", "QdError"]
