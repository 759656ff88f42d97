"""MI355X-native SSD layer (Mamba-2 structured state-space duality) forward and decode."""
