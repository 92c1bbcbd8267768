"""CPU fp64 oracle (test infrastructure only; see oracle.oracle)."""
from .oracle import (allowed, allowed_full_diagonal, allowed_pair_counts, attn_dense, attn_rows,
                     closed_form_pairs, count_pairs, doc_scores, rank, to_f64, token_tables)
