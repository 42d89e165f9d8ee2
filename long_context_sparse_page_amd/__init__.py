"""MI355X-native Locks decode path: page summaries, reconstructed-LSE page
scoring, GQA share-averaged top-k page selection and sparse paged
flash-decode, as hand-written HIP kernels for gfx950 behind a C ABI
(``include/locks.h``).  The Python side only marshals arguments."""
