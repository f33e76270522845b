"""MI355X-native DAMP decode step for Gated DeltaNet / Kimi Delta Attention recurrent states."""
