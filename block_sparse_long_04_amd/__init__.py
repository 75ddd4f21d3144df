"""Block-sparse causal prefill attention (FlashPrefill-style) for MI355X."""
