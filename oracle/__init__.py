"""Float64 CPU oracle of the VDA linear branch (test infrastructure only)."""
