"""MI355X-native canonical convolution (placeholder; the binding follows)."""
