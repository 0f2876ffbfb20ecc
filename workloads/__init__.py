"""Seeded synthetic workloads (input generation only; no attention arithmetic)."""
from .gen import *  # noqa: F401,F403
from .gen import CONFIGS, DecodeCase, PrefillCase, make_decode_case, make_prefill_case  # noqa: F401
