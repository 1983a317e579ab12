"""MI355X-native MoE layer forward pass (placeholder; the binding lands with the C ABI)."""
