"""MI355X-native fused softmax and LayerNorm row reductions (binding filled in below)."""
