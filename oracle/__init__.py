"""CPU oracle of the Stem sparse-prefill path (test infrastructure only)."""
