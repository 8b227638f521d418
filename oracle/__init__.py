"""fp64 CPU oracle (test infrastructure only; see rtp_oracle's header)."""
