"""MI355X-native draft-tree verify path (HIP kernels behind a C ABI)."""
