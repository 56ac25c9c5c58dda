"""Seeded synthetic inputs shared by the oracle tests and the HIP-path tests."""
