"""MI355X-native dense GEMM (placeholder until the binding lands)."""
