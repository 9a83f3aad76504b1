"""CPU oracle for the draft-tree build and verification: test infrastructure only."""
