"""Seeded synthetic inputs for the routed int4 MoE layer (shared by tests, smoke check and bench)."""
