// fa_merge.hip -- merge of two attention results over disjoint key sets by their row
// log-sum-exp, for gfx950 (MI355X).
//
// Method: the union of key sets A and B has lse = ln(e^lse_a + e^lse_b) and
// o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b. The "ascend-transformer-boost" article
// (场景四) splits multimodal attention into separate calls (text to text causally, text to
// image fully) whose results combine exactly this way.
//
// gfx950 mapping: a plain HBM stream (about 2 d + 2 elements read and d + 1 written per row
// of 16-bit data), so no LDS and no MFMA: each lane owns 16 contiguous bytes of a row (8
// 16-bit or 4 fp32 elements), the lanes of one row sit in one wave, and each reads both row
// statistics. In-place use (o == o_a, lse == lse_a) is safe: every lane reads its inputs
// before any lane of its row writes.
#include "fa_device.h"

namespace teaf {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_lse_kernel(const T *o_a, const float *lse_a,
                                                        const T *o_b, const float *lse_b, T *o,
                                                        float *lse, long rows)
{
    constexpr int PER = 16 / sizeof(T), LPR = D / PER;  // elements per lane, lanes per row
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    const long r = gid / LPR;
    const int part = (int)(gid % LPR);
    if (r >= rows) return;
    const float la = lse_a[r], lb = lse_b[r];
    const float m = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f, lm = -INFINITY;
    if (m != -INFINITY) {
        wa = fast_exp2((la - m) * kLog2e);
        wb = fast_exp2((lb - m) * kLog2e);
        const float t = wa + wb;
        lm = m + __builtin_amdgcn_logf(t) * kLn2;
        const float inv = 1.f / t;
        wa *= inv;
        wb *= inv;
    }
    typedef T vec __attribute__((ext_vector_type(PER)));
    const size_t at = (size_t)r * D + (size_t)part * PER;
    const vec a = *(const vec *)(o_a + at);
    const vec b = *(const vec *)(o_b + at);
    vec out;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        // a side with weight 0 contributes nothing, whatever its o holds
        const float x = wa == 0.f ? 0.f : wa * (float)a[e];
        const float y = wb == 0.f ? 0.f : wb * (float)b[e];
        out[e] = (T)(x + y);
    }
    *(vec *)(o + at) = out;
    if (part == 0) lse[r] = lm;
}

template <typename T, int D>
hipError_t launch_merge_t(const MergeArgs &a, hipStream_t s)
{
    constexpr int LPR = D / (16 / (int)sizeof(T));
    const long threads = a.rows * LPR;
    hipLaunchKernelGGL((merge_lse_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, (const T *)a.o_a, a.lse_a, (const T *)a.o_b, a.lse_b,
                       (T *)a.o, a.lse, a.rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t s)
{
    (void)hipGetLastError();
    if (a.dtype == 0) return a.d == 64 ? launch_merge_t<float, 64>(a, s) : launch_merge_t<float, 128>(a, s);
    if (a.dtype == 1)
        return a.d == 64 ? launch_merge_t<_Float16, 64>(a, s) : launch_merge_t<_Float16, 128>(a, s);
    return a.d == 64 ? launch_merge_t<__bf16, 64>(a, s) : launch_merge_t<__bf16, 128>(a, s);
}

}  // namespace teaf
