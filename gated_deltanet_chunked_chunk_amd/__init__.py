"""MI355X-native Gated DeltaNet chunked-prefill forward (placeholder; the
binding to the HIP library is added with the library)."""
