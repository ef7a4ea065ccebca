// kda_state_head.h -- the whole-head state pass (kda_state_head.hip) and the
// pipelined prefill that runs it beside the intra-chunk pass.  Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {

constexpr int kHeadThreads = 512;  // 8 waves per workgroup

struct StateHeadParams {
    const float *init_state;            // nullable (zeros); may equal final_state
    const int32_t *cu_seqlens, *chunk_offsets;
    float *o, *final_state;             // final_state nullable
    int64_t T;
    int32_t H, N;
    const char *ws;
    size_t pkg_bytes;
    PackageLayout L;
    int64_t c_begin, c_end;             // chunks [c_begin, c_end) of every sequence
};

// 64-token chunks, d_k = d_v = 128, fp16 package operands (the bf16 path).
hipError_t launch_state_head(const StateHeadParams &p, hipStream_t stream);

// The whole forward of one long sequence at those sizes (intra-chunk pass,
// this state pass, the layer's epilogue for gate mode 2), pipelined over
// segments on two CU-masked streams joined back to `stream`.  Returns
// hipErrorNotSupported, with nothing enqueued, for other calls (several or
// short sequences, more than 32 heads) or when CU-masked streams are
// unavailable.
hipError_t launch_prefill_pipelined(const PrefillArgs &a, hipStream_t stream);

}  // namespace kda
