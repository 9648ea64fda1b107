"""Exact, IO-aware attention forward for AMD Instinct MI355X (gfx950)."""
