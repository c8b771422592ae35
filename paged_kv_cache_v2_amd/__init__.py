"""MI355X-native paged single-query decode attention (V2 partition + LSE reduce, GQA)."""
