"""Workload presets and seeded synthetic inputs (no arithmetic of the forward pass)."""
