"""MI355X-native LapSum soft top-k (placeholder until the binding lands)."""
