"""MI355X-native paged decode attention (HIP for gfx950 behind a C-ABI)."""
