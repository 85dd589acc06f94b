/* vb_testing.h -- host-only helpers of libvbprop.so exported for its tests.
 *
 * These expose internal host-side decisions of the library so that CPU tests
 * can check them without a GPU.  They launch nothing, touch no device memory
 * and are not part of the bound-propagation interface (vb.h).
 */
#ifndef VB_TESTING_H
#define VB_TESTING_H

#include <stdint.h>

#include "vb.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Quotients x[i] / d for n values 0 <= x[i] < 2^31, computed the way the
 * kernels divide by a runtime constant: with the library's own multiply-high
 * magic numbers for d (the kernels evaluate the same multiply-high and shift).
 * mul and shr receive the magic numbers.  Returns 0, or -1 for d < 1, n < 0,
 * a NULL array or an x outside [0, 2^31). */
int32_t vb_testing_fastdiv(int32_t d, const int32_t* x, int64_t n, int32_t* q, uint32_t* mul, uint32_t* shr);

/* Width of the N-tiles the GEMM launcher picks for a 3x3, stride-1, pad-1
 * convolution from c_in to c_out channels on an h x w image: mode 0, 1 or 2
 * is its back-substitution over `rows` rows of Lambda with the store,
 * relaxation or concretisation epilogue (N = c_in); mode 4 is its forward
 * product over `rows` rows with the alpha-CROWN adjoint epilogue (N = c_out).
 * Returns the tile width (32, 64, 128 or 256), or -1 for bad arguments. */
int32_t vb_testing_conv_tile_n(int32_t mode, int32_t rows, int32_t h, int32_t w, int32_t c_in, int32_t c_out);

/* Which back-substitution the library uses for the identity rows over node
 * `start` down to the domain node `stop` (intermediate bounds): 0 dense rows
 * over every node, 1 footprint windows along a conv -> ReLU -> conv chain, 2
 * footprint windows through a region with residual additions.  -1 for a bad
 * graph or node indices. */
int32_t vb_testing_identity_path(const vb_graph* g, int32_t start, int32_t stop);

#ifdef __cplusplus
}
#endif

#endif /* VB_TESTING_H */
