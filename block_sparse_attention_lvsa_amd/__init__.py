"""MI355X-native LVSA frame-block-sparse attention (placeholder, filled in below)."""
