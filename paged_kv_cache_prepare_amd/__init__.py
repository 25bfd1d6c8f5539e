"""Paged KV-cache prepare + paged varlen attention for MI355X (gfx950)."""
