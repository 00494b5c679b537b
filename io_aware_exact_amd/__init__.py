"""Exact IO-aware attention forward for AMD MI355X (gfx950)."""
