"""Seeded synthetic inputs shared by the oracle and the GPU path (no method arithmetic)."""
from .inputs import *  # noqa: F401,F403
