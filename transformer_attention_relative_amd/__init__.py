"""MI355X-native fused relative-position attention forward (HIP, gfx950)."""
