"""MI355X-native hot path of a packed joint audio-video DiT block.

The compute lives in libh3dit.so (hand-written HIP for gfx950, C ABI in
include/h3dit.h); this package is the thin Python binding over it.
"""
from ._lib import H3Error, LIB_PATH, lib  # noqa: F401

__all__ = ["H3Error", "LIB_PATH", "lib", "ops"]


def __getattr__(name):
    # torch is imported only when the op wrappers are first used
    if name == "ops":
        import importlib
        return importlib.import_module(".ops", __name__)
    raise AttributeError(name)
