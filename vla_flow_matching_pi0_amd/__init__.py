"""MI355X-native flow-matching action expert (pi0.5-style denoise loop).

The compute path is libvfm.so (HIP kernels for gfx950 behind the C ABI in
include/vfm.h); `vfm` is its ctypes binding."""
