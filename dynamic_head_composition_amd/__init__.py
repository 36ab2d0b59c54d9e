"""Lightweight DC attention on MI355X: Python binding (placeholder until the library exists)."""
