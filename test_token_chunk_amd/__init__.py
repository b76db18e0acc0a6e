"""MI355X-native TTT-E2E inner loop (HIP/gfx950) behind a C ABI."""
