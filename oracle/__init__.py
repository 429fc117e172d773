"""CPU oracle for HGA routed attention: test infrastructure, never part of the product path."""
