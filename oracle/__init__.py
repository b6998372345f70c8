"""CPU oracle of the Prism attention path (test infrastructure only; see prism_oracle)."""
