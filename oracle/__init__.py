"""CPU float64 oracle of the GPT-2 training step (test infrastructure only)."""
