"""MI355X-native FlashAttention-2 exact attention (gfx950 HIP kernels behind a C ABI).

The library itself is ``libfa2.so`` (C ABI declared in ``include/fa2.h``); this
package only marshals arguments to it.  The library is loaded on first use.
"""
