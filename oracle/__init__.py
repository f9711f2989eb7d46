"""CPU oracle for the TurboQuant hot path -- test infrastructure only."""
