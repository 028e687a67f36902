"""MI355X-native sparse Mixture-of-Experts layer forward (HIP for gfx950)."""
