"""Placeholder; the binding is written next."""
