"""Batched speculative-decoding verify-and-accept on MI355X (gfx950)."""
