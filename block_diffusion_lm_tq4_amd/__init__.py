"""TQ4_1S dequantize-and-multiply library for MI355X (gfx950)."""
