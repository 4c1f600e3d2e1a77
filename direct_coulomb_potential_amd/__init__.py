"""cpmap: electrostatic potential maps on MI355X (gfx950)."""
