"""Seeded synthetic inputs shared by the oracle tests, the HIP parity tests and
the benchmark.  No attention arithmetic lives here."""
from .gen import *  # noqa: F401,F403
from .gen import DecodeCase, make_config, make_p3_case, make_random_case  # noqa: F401
