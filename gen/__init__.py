"""Seeded synthetic input generators shared by the oracle and the HIP path (no method arithmetic)."""
from .inputs import *  # noqa: F401,F403
