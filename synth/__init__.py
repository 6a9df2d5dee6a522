"""Seeded synthetic inputs shared by the GPU library's tests/benchmark and the
CPU oracle. Random numbers and casts only: no part of the recurrence lives here."""
from .inputs import *  # noqa: F401,F403
