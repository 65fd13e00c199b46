"""MI355X-native CSA / HCA hybrid compressed attention (binding to libcsa)."""
