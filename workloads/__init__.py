"""Seeded synthetic inputs for the paged-KV attention step (shared by the tests,
the benchmark and the smoke check).  Holds none of the method's arithmetic:
value streams, request shapes, block scattering and the serving-trace
scheduler that produces step shapes."""
from . import rng, configs  # noqa: F401
