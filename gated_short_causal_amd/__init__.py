"""MI355X-native LFM2 gated short causal convolution (ShortConv)."""
