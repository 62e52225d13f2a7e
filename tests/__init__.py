"""Tests: CPU oracle pins, ABI checks, and GPU parity against the oracle."""
