"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and rounds them to the storage
formats; it holds none of the scoring arithmetic.  See ``synth.inputs``."""
from .inputs import *  # noqa: F401,F403
