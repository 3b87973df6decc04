"""MI355X-native Faster Flash Decoding: fused sparse decode attention for long contexts."""
