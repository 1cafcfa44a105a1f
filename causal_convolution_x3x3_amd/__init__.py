"""MI355X-native chunked causal Conv3d decode (placeholder; the binding lands with the library)."""
