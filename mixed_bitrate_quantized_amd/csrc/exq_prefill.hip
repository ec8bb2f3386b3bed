// Prefill path (M > 16) for gfx950.  Interim version: runs the decode
// kernel over 16-row slices of x.
#include <hip/hip_runtime.h>

#include "exq_internal.h"

struct exq_layer;
extern exq_status exq_decode_rows(const exq_layer* L, const void* x, int M, void* y, hipStream_t stream);

exq_status exq_prefill_launch(const exq_layer* L, const void* x, int M, void* y, hipStream_t stream) {
    return exq_decode_rows(L, x, M, y, stream);
}
