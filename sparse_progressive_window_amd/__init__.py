"""MI355X-native progressive focused attention (PFA) layer chain."""
