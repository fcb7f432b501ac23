// synth_dev.hip -- device side of the seeded input generator (see synth_core.h).
// Built into libsynth_dev.so.  Fills a 16-bit buffer with the values the host
// generator gives for the same global indices.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_core.h"

namespace {

__global__ void __launch_bounds__(256) fill_kernel(uint16_t* __restrict__ out, int64_t n,
                                                   uint64_t first, uint64_t key, int64_t mult,
                                                   int e, int exp_bits, int frac_bits) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        out[j] = synth_value(key, first + (uint64_t)j, mult, e, exp_bits, frac_bits);
}

}  // namespace

extern "C" {

// Returns 0 on success, -1 on bad arguments, or the (positive) hipError_t of
// a failed launch.
int synth_dev_fill(void* out, int64_t n, uint64_t first, uint64_t key, int64_t mult, int32_t e,
                   int32_t exp_bits, int32_t frac_bits, void* stream) {
    if (n < 0 || (n > 0 && out == nullptr)) return -1;
    if (!(exp_bits == 5 && frac_bits == 10) && !(exp_bits == 8 && frac_bits == 7)) return -1;
    if (n == 0) return 0;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    uint16_t* o = (uint16_t*)out;
    int ei = e, eb = exp_bits, fb = frac_bits;
    void* args[] = {&o, &n, &first, &key, &mult, &ei, &eb, &fb};
    hipError_t err = hipLaunchKernel((const void*)fill_kernel, dim3((unsigned)blocks), dim3(256),
                                     args, 0, (hipStream_t)stream);
    return err == hipSuccess ? 0 : (int)err;
}

}  // extern "C"
