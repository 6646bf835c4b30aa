"""MI355X-native multi-token block-quantized mat-vec (Q8_0 / Q4_0 / BF16, T = 1..4)."""
