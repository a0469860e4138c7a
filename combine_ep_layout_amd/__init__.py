"""MI355X-native MoE expert-parallel layout / dispatch / combine (a world of one)."""
