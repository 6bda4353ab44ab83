"""MI355X-native jagged block attention (binding package; see binding.py)."""
