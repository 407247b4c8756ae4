"""CPU oracle (test infrastructure only). See moe_oracle.py."""
