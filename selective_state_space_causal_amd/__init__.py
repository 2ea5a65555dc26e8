"""MI355X-native selective state-space causal scan (prefill + decode) for one GPU channel slice."""
