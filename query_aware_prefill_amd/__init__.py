"""MI355X (gfx950) AI.IF join prefill: cascade attention over anchor KV
computed once, W8A16 decoder projections, and an 8-column head, behind the C
ABI in include/quail.h. ``binding`` is the thin ctypes layer; ``device``
uploads weights and allocates the pool/workspace with torch."""
from . import binding  # noqa: F401

__all__ = ["binding"]
