"""CPU oracle of the routed int4 MoE expert FFN (test infrastructure only)."""
