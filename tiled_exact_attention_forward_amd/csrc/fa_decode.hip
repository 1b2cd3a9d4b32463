// fa_decode.hip -- single-token attention against a paged K/V cache, for gfx950.
//
// Method: the cache is a pool of fixed pages of 256 tokens; a sequence's history is the
// chain of pages its page-table row names ("ascend-transformer-boost" article, 场景二, paged
// KV cache with page_size 256 and prefetch of the next K/V batch ahead of the math). The
// query is the newest token of its sequence and sees all of its keys.
//
// Decode is a matrix-vector product per (sequence, head): about one flop per byte of K/V,
// so it is bound by HBM bandwidth and uses plain vector FMAs, not the matrix cores.
// Split-KV: the split pass gives each workgroup 64 consecutive tokens (a quarter page,
// never crossing a page) of one sequence for 8 heads. A page stores [token][head][d], so
// those 8 heads of one token are 2 KB contiguous and every load instruction of a wave
// covers 1 KB contiguous. Each workgroup keeps an online softmax per head over its tokens
// and writes a partial output O_s (already divided by its own sum) and its log-sum-exp
// lse_s. The combine pass merges the splits of each (sequence, head):
//   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s,
// which equals attention over the union of the splits (the same identity that lets the
// multimodal case of the boost article split one attention into several calls).
// Slots past a sequence's length are never read, so stale or NaN cache contents there
// cannot leak into the result.
#include <math.h>

#include "fa_launch.h"

namespace teaf {
namespace {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kD = 128;        // head dimension
constexpr int kPage = 256;     // tokens per page
constexpr int kBatch = 8;      // tokens per thread kept in flight
constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ void to_float8(s16x8 x, float *f)
{
    if constexpr (sizeof(T) == 2 && __is_same(T, _Float16)) {
        const f16x8 h = __builtin_bit_cast(f16x8, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (float)h[e];
    } else {
        const bf16x8 h = __builtin_bit_cast(bf16x8, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (float)h[e];
    }
}

template <typename T>
__device__ __forceinline__ uint16_t from_float(float f)
{
    if constexpr (__is_same(T, _Float16)) return __builtin_bit_cast(uint16_t, (_Float16)f);
    else return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Sum over the 16 lanes of a row of the wave (lanes 16r .. 16r+15) with DPP moves.
__device__ __forceinline__ float row16_sum(float x)
{
    // quad_perm [1,0,3,2] and [2,3,0,1], then row_half_mirror and row_mirror.
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xb1, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4e, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xf, 0xf, true));
    return x;
}

// grid (max_splits, S, H / 8); 256 threads. Thread t: d chunk c = t % 16 (8 values),
// local head hl = (t / 16) % 8, token lane tl = t / 128 (tokens tl, tl + 2, ...).
template <typename T>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const uint16_t *__restrict__ Qp, const uint16_t *__restrict__ Kp,
    const uint16_t *__restrict__ Vp, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, float *__restrict__ part_o,
    float *__restrict__ part_lse, int H, int max_pages, int max_splits, float c)
{
    const int sp = blockIdx.x, s = blockIdx.y, hg = blockIdx.z;
    const int L = seq_lens[s];
    const int t0 = sp * kDecodeSplit;
    if (t0 >= L) return;  // workgroup-uniform
    const int tid = threadIdx.x;
    const int cc = tid & 15, hl = (tid >> 4) & 7, tl = tid >> 7;
    const int h = hg * kDecodeHeads + hl;
    const int ntok = min(kDecodeSplit, L - t0);
    const int page = page_table[(size_t)s * max_pages + t0 / kPage];
    const int slot0 = t0 % kPage;
    // element offset of (token slot0, head h, chunk cc) in the page pool
    const size_t base = (((size_t)page * kPage + slot0) * H + h) * kD + cc * 8;
    const size_t tstride = (size_t)H * kD;  // elements between consecutive tokens

    float q[8];
    to_float8<T>(*(const s16x8 *)(Qp + ((size_t)s * H + h) * kD + cc * 8), q);

    float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;

    for (int b0 = 0; b0 < kDecodeSplit; b0 += 2 * kBatch) {
        s16x8 kx[kBatch], vx[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int tt = b0 + tl + 2 * u;
            if (tt < ntok) {
                kx[u] = *(const s16x8 *)(Kp + base + tt * tstride);
                vx[u] = *(const s16x8 *)(Vp + base + tt * tstride);
            } else {
                kx[u] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
                vx[u] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
        float sc[kBatch];
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            float kf[8];
            to_float8<T>(kx[u], kf);
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf(q[e], kf[e], dot);
            dot = row16_sum(dot);
            const int tt = b0 + tl + 2 * u;
            sc[u] = tt < ntok ? dot * c : -INFINITY;
            mb = fmaxf(mb, sc[u]);
        }
        const float mn = fmaxf(m, mb);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = __builtin_amdgcn_exp2f(m - mu);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const float p = __builtin_amdgcn_exp2f(sc[u] - mu);
            l += p;
            float vf[8];
            to_float8<T>(vx[u], vf);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(p, vf[e], o[e]);
        }
    }

    // Merge the two token lanes (threads t and t + 128) through LDS.
    __shared__ float xm[128], xl[128], xo[128 * 9];
    if (tl == 1) {
        xm[tid - 128] = m;
        xl[tid - 128] = l;
#pragma unroll
        for (int e = 0; e < 8; ++e) xo[(tid - 128) * 9 + e] = o[e];
    }
    __syncthreads();
    if (tl == 0) {
        const float m1 = xm[tid], l1 = xl[tid];
        const float mn = fmaxf(m, m1);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float a0 = __builtin_amdgcn_exp2f(m - mu), a1 = __builtin_amdgcn_exp2f(m1 - mu);
        const float lt = l * a0 + l1 * a1;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const size_t slot = ((size_t)s * H + h) * max_splits + sp;
        float *po = part_o + slot * kD + cc * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) po[e] = (o[e] * a0 + xo[tid * 9 + e] * a1) * inv;
        if (cc == 0) part_lse[slot] = lt > 0.f ? mn + __builtin_amdgcn_logf(lt) : -INFINITY;
    }
}

// grid (S, H); 128 threads, one per output column. Partial lse values are in log2 units.
template <typename T>
__global__ __launch_bounds__(kD) void decode_combine_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse,
    const int32_t *__restrict__ seq_lens, uint16_t *__restrict__ O, float *__restrict__ LSE,
    int H, int max_splits)
{
    const int s = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
    const int ns = (seq_lens[s] + kDecodeSplit - 1) / kDecodeSplit;
    const size_t slot0 = ((size_t)s * H + h) * max_splits;
    float mx = -INFINITY;
    for (int i = 0; i < ns; ++i) mx = fmaxf(mx, part_lse[slot0 + i]);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float w = 0.f, acc = 0.f;
    for (int i = 0; i < ns; ++i) {
        const float a = __builtin_amdgcn_exp2f(part_lse[slot0 + i] - mu);
        w += a;
        acc = fmaf(a, part_o[(slot0 + i) * kD + d], acc);
    }
    O[((size_t)s * H + h) * kD + d] = from_float<T>(w > 0.f ? acc / w : 0.f);
    if (LSE != nullptr && d == 0)
        LSE[(size_t)s * H + h] = w > 0.f ? (mu + __builtin_amdgcn_logf(w)) * kLn2 : -INFINITY;
}

template <typename T>
hipError_t launch(const DecodeArgs &a, hipStream_t st)
{
    const int max_splits = decode_max_splits(a.max_pages, a.page_size);
    float *part_o = (float *)a.workspace;
    float *part_lse = part_o + (size_t)a.S * a.H * max_splits * kD;
    hipLaunchKernelGGL(decode_split_kernel<T>,
                       dim3((unsigned)max_splits, (unsigned)a.S, (unsigned)(a.H / kDecodeHeads)),
                       dim3(kThreads), 0, st, (const uint16_t *)a.q, (const uint16_t *)a.k_pages,
                       (const uint16_t *)a.v_pages, a.page_table, a.seq_lens, part_o, part_lse,
                       a.H, a.max_pages, max_splits, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel<T>, dim3((unsigned)a.S, (unsigned)a.H), dim3(kD), 0,
                       st, part_o, part_lse, a.seq_lens, (uint16_t *)a.o, a.lse, a.H, max_splits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st)
{
    (void)hipGetLastError();
    return a.dtype == 1 ? launch<_Float16>(a, st) : launch<__bf16>(a, st);
}

}  // namespace teaf
