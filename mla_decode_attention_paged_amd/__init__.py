"""Paged MLA decode attention for MI355X (gfx950)."""
