"""MI355X-native ROSA retrieval (placeholder; binding added with the C-ABI)."""
