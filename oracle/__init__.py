"""fp64 CPU oracle (test infrastructure only; see paged_ref's header)."""
