"""MI355X-native MLA latent-KV decode with a DSA lightning indexer (binding loaded lazily)."""
