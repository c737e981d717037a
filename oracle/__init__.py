"""CPU oracle for the W8A8 verify path (test infrastructure, never the product path)."""
