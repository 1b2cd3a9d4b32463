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
    const uint8_t *layout;  // block-sparse layout (mask 5), else null
};

// Block-sparse forward: mask id, tile edge and the largest key-block count a query block's
// visible-block list holds in LDS.
constexpr int kMaskBlockSparse = 5, kBlockSparseEdge = 128, kBlockSparseMaxKeyBlocks = 2048;

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

// Split pass of paged decode: one workgroup takes `split` consecutive tokens of one
// sequence (64, 128 or the whole 256-token page; a split never crosses a page). The host
// picks the largest split that still yields enough workgroups; the workspace is sized for
// the smallest, so it fits every choice.
constexpr int kDecodeMinSplit = 64;
// Heads of one workgroup of the split pass: 16 when H is a multiple of 16, else 8.
constexpr int kDecodeHeads = 8;

// Static scratch of the allocation-free decode (file-scope device array, one per GPU).
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;

inline int decode_workspace_splits(int max_pages, int page_size)
{
    long tokens = (long)max_pages * page_size;
    return (int)((tokens + kDecodeMinSplit - 1) / kDecodeMinSplit);
}

// Chunked prefill against a paged cache (pages of 256 tokens): q and o [S, Qmax, H, d],
// lse [S, Qmax, H]; sequence s's chunk is its newest q_lens[s] of seq_lens[s] tokens.
struct PrefillArgs {
    const void *q, *k_pages, *v_pages;
    const int32_t *page_table, *seq_lens, *q_lens;
    void *o;
    float *lse;
    int S, Qmax, H, d, max_pages, num_pages;
    float scale;
    int mask, window, n_global, dtype;
};

// Merge of two attention results over disjoint key sets: rows x d outputs (dtype) and row
// log-sum-exps (float32); o and lse may alias o_a and lse_a.
struct MergeArgs {
    const void *o_a;
    const float *lse_a;
    const void *o_b;
    const float *lse_b;
    void *o;
    float *lse;
    long rows;
    int d, dtype;
};

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    int B, H, Nq, Nkv, d;
    float scale;
    int mask, window, n_global, dtype;
    void *workspace;  // backward_workspace_floats(B, H, Nq) floats of row statistics
    const uint8_t *layout;  // block-sparse layout (mask 5), else null
};

// Row statistics of the backward: per 32-row tile of each (b, h), 32 log2-scaled LSE values
// then 32 values of -D, D = rowsum(dO o O).
inline size_t backward_workspace_floats(int B, int H, int Nq)
{
    return (size_t)B * H * (size_t)((Nq + 31) / 32) * 64;
}

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream);
hipError_t launch_backward(const BwdArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// Bytes of split partials launch_decode places in a.workspace for these arguments (never
// more than the workspace size fa_decode_paged_workspace_bytes reports).
size_t decode_partials_bytes(const DecodeArgs &a);
// Device address of the decode's static scratch on the device `stream` runs on.
hipError_t decode_static_scratch(hipStream_t stream, void **ptr);
hipError_t launch_prefill_paged(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs &a, hipStream_t stream);
// Causal forward (16-bit types) whose keys are [0, n1) from a.k/a.v ([B,H,n1,d]) and
// [n1, a.Nkv) from k2/v2 ([B,H,a.Nkv-n1,d]); n1 a multiple of 32.
hipError_t launch_forward_causal_two_part(const FwdArgs &a, const void *k2, const void *v2,
                                         int n1, hipStream_t stream);

}  // namespace teaf
