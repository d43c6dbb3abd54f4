"""MI355X-native forward pass of VideoNSA's hybrid attention layer."""
