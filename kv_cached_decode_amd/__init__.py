"""kv_cached_decode_amd -- KV-cached decode attention for MI355X (gfx950)."""
