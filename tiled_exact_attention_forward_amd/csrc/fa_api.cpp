// fa_api.cpp -- the C ABI of libteaf.so: host-side argument checks, then one launch call.
// Every check runs before anything is enqueued, so a rejected call writes nothing.
#include <limits.h>
#include <stdint.h>

#include <algorithm>

#include "fa.h"
#include "fa_bwd32.h"
#include "fa_launch.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Workgroups of a one-dimensional launch of 256-thread workgroups: a dispatch counts its
// grid in work-items with 32 bits.
constexpr long long kMaxWorkgroups1D = (1ll << 32) / 256 - 1;

// Workgroups of the merge launch: 16 bytes of a row per thread.
long long merge_workgroups(long long rows, int d, int elem)
{
    return (rows * (d * elem / 16) + 255) / 256;
}

thread_local hipError_t g_last_hip = hipSuccess;

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return FA_OK;
    g_last_hip = e;
    return FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_version(void) { return 1 * 10000 + 0 * 100 + 0; }

const char *fa_last_hip_error(void) { return hipGetErrorString(g_last_hip); }

const char *fa_status_string(int status)
{
    switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "a size argument is out of range";
    case FA_ERR_UNSUPPORTED: return "valid arguments that the library does not support";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "the HIP runtime rejected a launch";
    case FA_ERR_SCRATCH:
        return "the call needs more scratch than the library's static array holds";
    default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// Checks of one forward call; on success fills *a (window and prefix counts clamped).
int check_forward(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                  int H, int Nq, int Nkv, int d, float scale, int mask_mode, int window,
                  int n_global, int dtype, teaf::FwdArgs *a)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || Nq < 1 || Nkv < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (mask_mode < FA_MASK_NONE || mask_mode > FA_MASK_PREFIX_LM) return FA_ERR_UNSUPPORTED;
    if (mask_mode == FA_MASK_WINDOW_GLOBAL && (window < 1 || n_global < 0)) return FA_ERR_SHAPE;
    if (mask_mode == FA_MASK_BAND && window < 0) return FA_ERR_SHAPE;
    if (mask_mode == FA_MASK_PREFIX_LM && n_global < 0) return FA_ERR_SHAPE;
    const long long bh = (long long)B * H;
    const long long nqt = (Nq + 127) / 128;
    if (bh * nqt > kMaxWorkgroups1D) return FA_ERR_SHAPE;
    if ((long long)Nq * d > (long long)INT_MAX || (long long)Nkv * d > (long long)INT_MAX)
        return FA_ERR_SHAPE;
    if (!(scale == scale)) return FA_ERR_SHAPE;  // NaN scale
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return FA_ERR_UNSUPPORTED;
    // Window and global/prefix counts beyond Nq + Nkv and Nkv change nothing; clamping them
    // keeps the kernels' position arithmetic inside int.
    const bool uses_w = mask_mode == FA_MASK_WINDOW_GLOBAL || mask_mode == FA_MASK_BAND;
    const bool uses_g = mask_mode == FA_MASK_WINDOW_GLOBAL || mask_mode == FA_MASK_PREFIX_LM;
    const int wc = uses_w ? (int)std::min<long long>(window, (long long)Nq + Nkv) : 0;
    const int gc = uses_g ? std::min(n_global, Nkv) : 0;
    *a = teaf::FwdArgs{q, k, v, o, lse, B, H, Nq, Nkv, d, scale, mask_mode, wc, gc, dtype};
    return FA_OK;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t elem_bytes(int dtype) { return dtype == FA_F32 ? 4 : 2; }

}  // namespace

extern "C" {

int fa_forward(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
               int Nq, int Nkv, int d, float scale, int mask_mode, int window, int n_global,
               int dtype, void *stream)
{
    teaf::FwdArgs a;
    const int st = check_forward(q, k, v, o, lse, B, H, Nq, Nkv, d, scale, mask_mode, window,
                                 n_global, dtype, &a);
    if (st != FA_OK) return st;
    return hip_status(teaf::launch_forward(a, (hipStream_t)stream));
}

int fa_merge_lse(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b,
                 void *o, float *lse, long long rows, int d, int dtype, void *stream)
{
    if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse) return FA_ERR_NULL;
    if (rows < 1 || rows > (1ll << 40)) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (merge_workgroups(rows, d, (int)elem_bytes(dtype)) > kMaxWorkgroups1D) return FA_ERR_SHAPE;
    if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o)) return FA_ERR_UNSUPPORTED;
    teaf::MergeArgs a{o_a, lse_a, o_b, lse_b, o, lse, (long)rows, d, dtype};
    return hip_status(teaf::launch_merge(a, (hipStream_t)stream));
}

size_t fa_multimodal_workspace_bytes(int B, int H, int n_txt, int d, int dtype)
{
    if (B < 1 || H < 1 || n_txt < 1 || d < 1) return 0;
    const size_t rows = (size_t)B * H * n_txt;
    return align256(rows * d * elem_bytes(dtype)) + rows * sizeof(float);
}

int fa_multimodal_forward(const void *q_img, const void *k_img, const void *v_img,
                          const void *q_txt, const void *k_txt, const void *v_txt, void *o_img,
                          float *lse_img, void *o_txt, float *lse_txt, int B, int H, int n_img,
                          int n_txt, int d, float scale, int dtype, int text_mode,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    teaf::FwdArgs img, txt, cross;
    int st = check_forward(q_img, k_img, v_img, o_img, lse_img, B, H, n_img, n_img, d, scale,
                           FA_MASK_NONE, 0, 0, dtype, &img);
    if (st != FA_OK) return st;
    st = check_forward(q_txt, k_txt, v_txt, o_txt, lse_txt, B, H, n_txt, n_txt, d, scale,
                       FA_MASK_CAUSAL, 0, 0, dtype, &txt);
    if (st != FA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (text_mode == FA_MULTIMODAL_FUSED) {
        // text rows against [image; text] keys, causal with bottom-right alignment: every
        // image key, and text keys up to the row's own position
        if (n_img % 32 != 0 || dtype == FA_F32) return FA_ERR_UNSUPPORTED;
        if ((long long)(n_img + (long long)n_txt) * d > (long long)INT_MAX) return FA_ERR_SHAPE;
        teaf::FwdArgs fused = txt;
        fused.k = k_img;
        fused.v = v_img;
        fused.Nkv = n_img + n_txt;
        hipError_t e = teaf::launch_forward(img, s);
        if (e == hipSuccess) e = teaf::launch_forward_causal_two_part(fused, k_txt, v_txt, n_img, s);
        return hip_status(e);
    }
    if (text_mode != FA_MULTIMODAL_SPLIT_MERGE) return FA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < fa_multimodal_workspace_bytes(B, H, n_txt, d, dtype) ||
        !aligned16(workspace))
        return FA_ERR_WORKSPACE;
    const size_t rows = (size_t)B * H * n_txt;
    if (merge_workgroups((long long)rows, d, (int)elem_bytes(dtype)) > kMaxWorkgroups1D)
        return FA_ERR_SHAPE;
    char *ws = (char *)workspace;
    float *lse_x = (float *)(ws + align256(rows * d * elem_bytes(dtype)));
    st = check_forward(q_txt, k_img, v_img, ws, lse_x, B, H, n_txt, n_img, d, scale,
                       FA_MASK_NONE, 0, 0, dtype, &cross);
    if (st != FA_OK) return st;
    const teaf::MergeArgs mg{o_txt, lse_txt, ws, lse_x, o_txt, lse_txt, (long)rows, d, dtype};
    hipError_t e = teaf::launch_forward(img, s);
    if (e == hipSuccess) e = teaf::launch_forward(txt, s);
    if (e == hipSuccess) e = teaf::launch_forward(cross, s);
    if (e == hipSuccess) e = teaf::launch_merge(mg, s);
    return hip_status(e);
}

int fa_forward_block_sparse(const void *q, const void *k, const void *v, void *o, float *lse,
                            int B, int H, int Nq, int Nkv, int d, float scale,
                            const uint8_t *layout, int block, int dtype, void *stream)
{
    if (!q || !k || !v || !o || !lse || !layout) return FA_ERR_NULL;
    if (B < 1 || H < 1 || Nq < 1 || Nkv < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (block != teaf::kBlockSparseEdge) return FA_ERR_UNSUPPORTED;
    if ((long long)Nkv > (long long)teaf::kBlockSparseMaxKeyBlocks * teaf::kBlockSparseEdge)
        return FA_ERR_UNSUPPORTED;
    const long long bh = (long long)B * H;
    const long long nqt = (Nq + 127) / 128;
    if (bh * nqt > kMaxWorkgroups1D) return FA_ERR_SHAPE;
    if ((long long)Nq * d > (long long)INT_MAX || (long long)Nkv * d > (long long)INT_MAX)
        return FA_ERR_SHAPE;
    if (!(scale == scale)) return FA_ERR_SHAPE;  // NaN scale
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return FA_ERR_UNSUPPORTED;
    teaf::FwdArgs a{q, k, v, o, lse, B, H, Nq, Nkv, d, scale, teaf::kMaskBlockSparse, 0, 0,
                    dtype, layout};
    return hip_status(teaf::launch_forward(a, (hipStream_t)stream));
}

size_t fa_backward_workspace_bytes(int B, int H, int Nq)
{
    if (B < 1 || H < 1 || Nq < 1) return 0;
    return teaf::backward_workspace_floats(B, H, Nq) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks shared by the backward entry points (all but the mask arguments).
int check_backward(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dout, void *dq, void *dk, void *dv, int B, int H, int Nq, int Nkv,
                   int d, float scale, int dtype, void *workspace, size_t workspace_bytes)
{
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
    if (B < 1 || H < 1 || Nq < 1 || Nkv < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    const long long bh = (long long)B * H;
    if (bh * ((Nq + 127) / 128) > kMaxWorkgroups1D || bh * ((Nkv + 127) / 128) > kMaxWorkgroups1D)
        return FA_ERR_SHAPE;
    if ((long long)Nq * d > (long long)INT_MAX || (long long)Nkv * d > (long long)INT_MAX)
        return FA_ERR_SHAPE;
    if (!(scale == scale)) return FA_ERR_SHAPE;
    if (!workspace || workspace_bytes < fa_backward_workspace_bytes(B, H, Nq))
        return FA_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// The float32 backward has kernels of its own (fp32 products throughout).
hipError_t launch_backward_any(const teaf::BwdArgs &a, hipStream_t s)
{
    return a.dtype == FA_F32 ? teaf::launch_backward32(a, s) : teaf::launch_backward(a, s);
}

}  // namespace

extern "C" {

int fa_backward(const void *q, const void *k, const void *v, const void *o, const float *lse,
                const void *dout, void *dq, void *dk, void *dv, int B, int H, int Nq, int Nkv,
                int d, float scale, int mask_mode, int window, int n_global, int dtype,
                void *workspace, size_t workspace_bytes, void *stream)
{
    const int st = check_backward(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nkv, d, scale,
                                  dtype, workspace, workspace_bytes);
    if (st != FA_OK) return st;
    if (mask_mode < FA_MASK_NONE || mask_mode > FA_MASK_PREFIX_LM) return FA_ERR_UNSUPPORTED;
    if (mask_mode == FA_MASK_WINDOW_GLOBAL && (window < 1 || n_global < 0)) return FA_ERR_SHAPE;
    if (mask_mode == FA_MASK_BAND && window < 0) return FA_ERR_SHAPE;
    if (mask_mode == FA_MASK_PREFIX_LM && n_global < 0) return FA_ERR_SHAPE;
    const bool uses_w = mask_mode == FA_MASK_WINDOW_GLOBAL || mask_mode == FA_MASK_BAND;
    const bool uses_g = mask_mode == FA_MASK_WINDOW_GLOBAL || mask_mode == FA_MASK_PREFIX_LM;
    const int wc = uses_w ? (int)std::min<long long>(window, (long long)Nq + Nkv) : 0;
    const int gc = uses_g ? std::min(n_global, Nkv) : 0;
    teaf::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nkv, d, scale, mask_mode, wc,
                    gc, dtype, workspace, nullptr};
    return hip_status(launch_backward_any(a, (hipStream_t)stream));
}

int fa_backward_block_sparse(const void *q, const void *k, const void *v, const void *o,
                             const float *lse, const void *dout, void *dq, void *dk, void *dv,
                             int B, int H, int Nq, int Nkv, int d, float scale,
                             const uint8_t *layout, int block, int dtype, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    const int st = check_backward(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nkv, d, scale,
                                  dtype, workspace, workspace_bytes);
    if (st != FA_OK) return st;
    if (!layout) return FA_ERR_NULL;
    if (block != teaf::kBlockSparseEdge) return FA_ERR_UNSUPPORTED;
    const long long most = (long long)teaf::kBlockSparseMaxKeyBlocks * teaf::kBlockSparseEdge;
    if ((long long)Nq > most || (long long)Nkv > most) return FA_ERR_UNSUPPORTED;
    teaf::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nkv, d, scale,
                    teaf::kMaskBlockSparse, 0, 0, dtype, workspace, layout};
    return hip_status(launch_backward_any(a, (hipStream_t)stream));
}

int fa_prefill_paged(const void *q, const void *k_pages, const void *v_pages,
                     const int32_t *page_table, const int32_t *seq_lens, const int32_t *q_lens,
                     void *o, float *lse, int page_size, int num_seqs, int Qmax, int H, int d,
                     int max_pages_per_seq, int num_pages, float scale, int mask_mode,
                     int window, int n_global, int dtype, void *stream)
{
    if (!q || !k_pages || !v_pages || !page_table || !seq_lens || !q_lens || !o || !lse)
        return FA_ERR_NULL;
    if (num_seqs < 1 || Qmax < 1 || H < 1 || max_pages_per_seq < 1 || num_pages < 1 ||
        page_size < 1)
        return FA_ERR_SHAPE;
    if (page_size != 256 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (mask_mode < FA_MASK_NONE || mask_mode > FA_MASK_PREFIX_LM) return FA_ERR_UNSUPPORTED;
    if (mask_mode == FA_MASK_WINDOW_GLOBAL && (window < 1 || n_global < 0)) return FA_ERR_SHAPE;
    if (mask_mode == FA_MASK_BAND && window < 0) return FA_ERR_SHAPE;
    if (mask_mode == FA_MASK_PREFIX_LM && n_global < 0) return FA_ERR_SHAPE;
    if (H > 65535 || (long long)max_pages_per_seq * page_size > (1ll << 30)) return FA_ERR_SHAPE;
    if ((long long)num_seqs * H * ((Qmax + 127) / 128) > kMaxWorkgroups1D) return FA_ERR_SHAPE;
    if (!(scale == scale)) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o))
        return FA_ERR_UNSUPPORTED;
    const bool uses_w = mask_mode == FA_MASK_WINDOW_GLOBAL || mask_mode == FA_MASK_BAND;
    const bool uses_g = mask_mode == FA_MASK_WINDOW_GLOBAL || mask_mode == FA_MASK_PREFIX_LM;
    const int wc = uses_w ? std::min(window, 1 << 30) : 0;
    const int gc = uses_g ? std::min(n_global, max_pages_per_seq * page_size) : 0;
    teaf::PrefillArgs a{q, k_pages, v_pages, page_table, seq_lens, q_lens, o, lse, num_seqs,
                        Qmax, H, d, max_pages_per_seq, num_pages, scale, mask_mode, wc, gc,
                        dtype};
    return hip_status(teaf::launch_prefill_paged(a, (hipStream_t)stream));
}

size_t fa_decode_paged_workspace_bytes(int num_seqs, int H, int d, int max_pages_per_seq,
                                       int page_size)
{
    if (num_seqs < 1 || H < 1 || d < 1 || max_pages_per_seq < 1 || page_size < 1) return 0;
    const size_t splits = (size_t)teaf::decode_workspace_splits(max_pages_per_seq, page_size);
    return (size_t)num_seqs * H * splits * ((size_t)d + 1) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks shared by the two decode entry points (everything but the scratch memory); on
// success fills *a with a null workspace.
int check_decode(const void *q, const void *k_pages, const void *v_pages,
                 const int32_t *page_table, const int32_t *seq_lens, void *o, float *lse,
                 int page_size, int num_seqs, int H, int d, int max_pages_per_seq, int num_pages,
                 float scale, int dtype, teaf::DecodeArgs *a)
{
    if (!q || !k_pages || !v_pages || !page_table || !seq_lens || !o) return FA_ERR_NULL;
    if (num_seqs < 1 || H < 1 || max_pages_per_seq < 1 || num_pages < 1 || page_size < 1)
        return FA_ERR_SHAPE;
    if (page_size != 256 || d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (H % teaf::kDecodeHeads != 0) return FA_ERR_UNSUPPORTED;
    // Launch grids: the split pass is (H / heads, splits, num_seqs), where the splits of the
    // longest sequence the table allows number max_pages_per_seq whenever there are more
    // than 2048 of them (one per 256-token page); the combine pass is (num_seqs, H). A grid
    // dimension past x takes at most 65535.
    if (num_seqs > 65535 || H > 65535 || max_pages_per_seq > 65535) return FA_ERR_SHAPE;
    if ((long long)num_pages * page_size * H * d > (long long)1 << 40) return FA_ERR_SHAPE;
    if ((long long)max_pages_per_seq * page_size > (1ll << 30)) return FA_ERR_SHAPE;
    if (!(scale == scale)) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o))
        return FA_ERR_UNSUPPORTED;
    *a = teaf::DecodeArgs{q, k_pages, v_pages, page_table, seq_lens, o, lse, page_size,
                          num_seqs, H, d, max_pages_per_seq, num_pages, scale, dtype, nullptr};
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                    const int32_t *page_table, const int32_t *seq_lens, void *o, float *lse,
                    int page_size, int num_seqs, int H, int d, int max_pages_per_seq,
                    int num_pages, float scale, int dtype, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    teaf::DecodeArgs a;
    const int rc = check_decode(q, k_pages, v_pages, page_table, seq_lens, o, lse, page_size,
                                num_seqs, H, d, max_pages_per_seq, num_pages, scale, dtype, &a);
    if (rc != FA_OK) return rc;
    const size_t need =
        fa_decode_paged_workspace_bytes(num_seqs, H, d, max_pages_per_seq, page_size);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_WORKSPACE;
    a.workspace = workspace;
    return hip_status(teaf::launch_decode(a, (hipStream_t)stream));
}

int fa_decode_paged_noalloc(const void *q, const void *k_pages, const void *v_pages,
                            const int32_t *page_table, const int32_t *seq_lens, void *o,
                            float *lse, int page_size, int num_seqs, int H, int d,
                            int max_pages_per_seq, int num_pages, float scale, int dtype,
                            void *stream)
{
    teaf::DecodeArgs a;
    const int rc = check_decode(q, k_pages, v_pages, page_table, seq_lens, o, lse, page_size,
                                num_seqs, H, d, max_pages_per_seq, num_pages, scale, dtype, &a);
    if (rc != FA_OK) return rc;
    if (teaf::decode_partials_bytes(a) > teaf::kDecodeScratchBytes) return FA_ERR_SCRATCH;
    const hipError_t e = teaf::decode_static_scratch((hipStream_t)stream, &a.workspace);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(teaf::launch_decode(a, (hipStream_t)stream));
}

}  // extern "C"
