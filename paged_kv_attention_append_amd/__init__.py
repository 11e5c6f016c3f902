"""Paged-KV attention with slot-mapped append for AMD MI355X (gfx950)."""
