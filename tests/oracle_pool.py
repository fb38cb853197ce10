"""Parallel host generation of the experts the oracle needs (re-exported from
``moe_inputs.host_cache``: a spawn pool of numpy workers that never touch
the GPU)."""
from __future__ import annotations

from moe_inputs.host_cache import prefetch, shutdown  # noqa: F401
