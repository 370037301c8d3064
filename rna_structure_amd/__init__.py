"""FlashIPA forward for MI355X (gfx950): lifted invariant point attention on
hand-written HIP kernels behind a C ABI (include/flashipa.h)."""
from . import synth  # noqa: F401

__all__ = ["synth", "load", "FlashIPA", "forward", "device_inputs"]


def __getattr__(name):
    if name in ("load", "FlashIPA", "forward", "device_inputs"):
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
