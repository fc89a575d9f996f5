"""Placeholder; the binding is filled in with the HIP library."""
