"""fp64 CPU oracle of the Mamba-3 SSM core (test infrastructure only)."""
