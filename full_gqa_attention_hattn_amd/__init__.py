"""MI355X-native hybrid GQA attention layer (Spark-X2.5/X2.6-4B): HIP kernels behind the
C ABI of include/hattn.h, and a thin ctypes binding (``hattn``) over it."""
