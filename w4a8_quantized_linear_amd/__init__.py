"""MI355X-native W4A8 quantized linear layer (placeholder; binding added with the library)."""
