"""CPU oracle of the routed MoE FFN layer -- test infrastructure only."""
