"""fp64 CPU oracle: test infrastructure only (see kv8_oracle's header)."""
