"""Seeded synthetic inputs shared by the tests, the oracle checks and bench.py."""
