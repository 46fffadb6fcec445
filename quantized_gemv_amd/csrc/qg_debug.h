// qg_debug.h -- device-side checks of the outlier path, run after the
// outlier split and the outlier-column gather when the environment holds
// QG_DEBUG=1.  They only read: the index list as the kernels received it,
// and the outputs of the kernels just launched.  A failed check sets a bit
// of a per-device flag word, which the host reads (after synchronizing the
// stream) and clears.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_launch.h"

namespace qg {

enum : uint32_t {
    kDbgIdx = 1u,     // an index out of [0, cols) or not above the one before it
    kDbgSplit = 2u,   // a gathered outlier activation differs from x, a code at an outlier column is not 0,
                      // or a padding column of x_out is not 0
    kDbgGather = 4u,  // a gathered weight differs from bf16(w), or a padding column is not 0
};

// Checks of qg_quantize_absmax_split's outputs (q [rows][cols], x_out [rows][ld]).
// selftest: expect every gathered value with its lowest bit flipped (a
// correct call with outliers then fails its check)
hipError_t debug_check_split(const uint16_t* x, int64_t rows, int64_t cols, const OutlierIdx& idx, int n_out,
                             const int8_t* q, const uint16_t* x_out, int ld, bool selftest, hipStream_t st);
// Checks of qg_gather_columns_bf16's output (w_out [n][ld]).
hipError_t debug_check_gather(const float* w, int64_t n, int64_t k, const OutlierIdx& idx, int n_out,
                              const uint16_t* w_out, int ld, bool selftest, hipStream_t st);
// Waits for the stream, returns the flag word of the current device in
// *flags and clears it.  Not usable while the stream is being captured.
hipError_t debug_take_flags(hipStream_t st, uint32_t* flags);

}  // namespace qg
