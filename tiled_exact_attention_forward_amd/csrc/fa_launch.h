// Internal launch interface between the C ABI layer (fa_api.cpp) and the HIP kernel files.
// Arguments have been validated by the caller; these only pick an instantiation and launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace teaf {

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, H, Nq, Nkv, d;
    float scale;
    int mask, window, n_global, dtype;
};

struct DecodeArgs {
    const void *q, *k_pages, *v_pages;
    const int32_t *page_table, *seq_lens;
    void *o;
    float *lse;
    int page_size, S, H, d, max_pages, num_pages;
    float scale;
    int dtype;
    void *workspace;
};

// Tokens of one sequence handled by one workgroup of the split pass.
constexpr int kDecodeSplit = 64;
// Heads handled by one workgroup of the split pass.
constexpr int kDecodeHeads = 8;

inline int decode_max_splits(int max_pages, int page_size)
{
    long tokens = (long)max_pages * page_size;
    return (int)((tokens + kDecodeSplit - 1) / kDecodeSplit);
}

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace teaf
