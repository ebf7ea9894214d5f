"""MI355X-native CSA2 layer hot path: the libcsa2 C-ABI library and its Python binding."""
