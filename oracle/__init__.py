"""fp64 CPU oracle of the exact attention forward. Test infrastructure only."""
