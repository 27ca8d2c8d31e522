"""additive_bias_gqa_amd: additive-bias GQA attention over an external static KV
cache, for MI355X (gfx950)."""
