"""MI355X-native fused scaled-dot-product attention (placeholder during bring-up)."""
