"""MI355X-native Gated Residual read/write path (binding filled in below)."""
