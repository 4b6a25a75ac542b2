"""MI355X-native accelerator linear layer (placeholder; binding added below)."""
