"""MI355X-native fused attention forward (placeholder while the binding is written)."""
