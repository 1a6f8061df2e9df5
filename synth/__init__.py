"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check."""
from .inputs import CONFIGS, Config, generate, make_inputs  # noqa: F401
