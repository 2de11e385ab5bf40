"""CPU oracle (test infrastructure only): see ``oracle.vsa_oracle``."""
