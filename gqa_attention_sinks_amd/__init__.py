"""Grouped-query flash attention with per-head learned sinks for MI355X (gfx950).

``workloads`` holds the seeded input generators.
"""
