"""MI355X-native FlashAdamW step (bit-companded Adam): a C-ABI HIP library
(``libflashopt.so``) and a thin ctypes binding with the same entry-point names."""
