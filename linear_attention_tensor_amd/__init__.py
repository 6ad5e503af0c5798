"""Tensor Cache outer-product memory for MI355X (gfx950).

The compute runs in the HIP library ``libtc.so`` (C ABI declared in
``include/tc.h``); ``ops`` marshals torch tensors into it.  Importing this
package does not load the library; the first op call does, and it raises if
the library is missing.
"""
__version__ = "0.1.0"
