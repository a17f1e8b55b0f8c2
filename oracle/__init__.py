"""Float64 CPU oracle (test infrastructure only; see gdn_ref's header)."""
