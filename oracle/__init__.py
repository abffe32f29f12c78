"""CPU oracle (test infrastructure only): see dflash_oracle."""
