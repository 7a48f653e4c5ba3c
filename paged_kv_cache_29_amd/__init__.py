"""Paged decode attention for MI355X (gfx950)."""
