"""FP64 CPU oracle (test infrastructure; see ``oracle.linear_logp``)."""
