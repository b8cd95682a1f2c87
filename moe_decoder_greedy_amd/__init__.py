"""MI355X-native FastMTP verify step through a Jina-OCR-v1 style MoE decoder.

The computation lives in libmoev.so (HIP kernels for gfx950 behind the C ABI in
include/moev.h).  ``ops`` binds each entry point; ``model.DeviceModel`` keeps a
synthetic decoder resident in HBM and runs whole verify steps.  Importing
``ops`` or ``model`` loads the library and raises if it has not been built
(``python -m moe_decoder_greedy_amd.build``).
"""
__version__ = "0.1.0"
