"""MI355X-native FlashAdamW step (bit-companded Adam): a C-ABI HIP library
(``libflashopt.so``, built from ``csrc/``) and a thin ctypes binding with the
same entry-point names (``flashopt``)."""
from . import flashopt  # noqa: F401  (the library itself loads at first use)
