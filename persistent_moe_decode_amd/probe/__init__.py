"""Streaming-read probe (measurement tool; not part of the decode path)."""
