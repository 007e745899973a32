"""MI355X (gfx950) paged GQA decode + per-block scoring.

The compute lives in the HIP library ``libkvs.so`` (C ABI in include/kvs.h);
``api`` is its Python binding and ``session`` the device-memory plumbing
that runs one decode + scoring step over a materialised workload.
"""
from . import api  # noqa: F401
from .api import KvsError  # noqa: F401
