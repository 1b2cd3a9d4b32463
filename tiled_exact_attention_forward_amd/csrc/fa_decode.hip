// fa_decode.hip -- single-token attention against a paged K/V cache, for gfx950.
//
// Method: the cache is a pool of fixed pages of 256 tokens; a sequence's history is the
// chain of pages its page-table row names ("ascend-transformer-boost" article, 场景二, paged
// KV cache with page_size 256 and prefetch of the next K/V batch ahead of the math). The
// query is the newest token of its sequence and sees all of its keys.
//
// Decode is a matrix-vector product per (sequence, head): about one flop per byte of K/V,
// so it is bound by HBM bandwidth and uses plain vector FMAs, not the matrix cores.
// Split-KV: the split pass gives each workgroup a run of consecutive tokens of one
// sequence (64, 128 or a whole 256-token page, never crossing a page) for 16 heads (8 if H
// is not a multiple of 16). A page stores [token][head][d], so those heads of one token
// are contiguous (4 KB for 16 heads) and every wave-wide load covers 1 KB. K and V stream
// through non-temporal loads one batch of tokens ahead of the math. Each workgroup keeps an
// online softmax per head over its tokens and writes a partial output O_s (already divided
// by its own sum) and its log-sum-exp lse_s. The combine pass merges the splits of each
// (sequence, head):
//   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s,
// which equals attention over the union of the splits (the same identity that lets the
// multimodal case of the boost article split one attention into several calls).
// Slots past a sequence's length are never read, so stale or NaN cache contents there
// cannot leak into the result.
#include <math.h>

#include <mutex>

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

// K/V are read once per call: non-temporal loads stream them past the caches.
__device__ __forceinline__ s16x8 stream_load(const uint16_t *p)
{
    return __builtin_nontemporal_load((const s16x8 *)p);
}

// Split pass. grid (H / HW, max_splits, S), 256 threads; a workgroup owns SPLIT
// consecutive tokens (inside one page) of one sequence for HW heads. A page stores
// [token][head][d], so the HW heads of one token are HW * 256 bytes contiguous: thread t
// reads 16-byte chunk t % 16 of head (t / 16) % HW, and each wave-wide load covers 1 KB
// contiguous.
//   HW = 16: one head per thread, all 256 threads on one token;
//   HW = 8 : one head per thread, two token lanes (tokens tl, tl + 2, ...).
// Loads run one batch of tokens ahead of the math (two register buffers). The page id is
// clamped into the pool, so a corrupt table entry gives wrong values but never a read
// outside the pool (as in the chunked prefill).
template <typename T, int HW, int SPLIT>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const uint16_t *__restrict__ Qp, const uint16_t *__restrict__ Kp,
    const uint16_t *__restrict__ Vp, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, float *__restrict__ part_o,
    float *__restrict__ part_lse, int H, int max_pages, int num_pages, int max_splits, float c)
{
    constexpr int PAIRS = HW * 16;                       // (head, chunk) pairs per token
    constexpr int HPT = PAIRS > kThreads ? PAIRS / kThreads : 1;   // heads per thread
    constexpr int TL = PAIRS < kThreads ? kThreads / PAIRS : 1;    // token lanes
    constexpr int B = 4;                                 // tokens per lane per batch
    constexpr int NB = SPLIT / (B * TL);                 // batches per split
    static_assert(NB % 2 == 0, "batches are processed in pairs");

    const int hg = blockIdx.x, sp = blockIdx.y, s = blockIdx.z;
    const int L = seq_lens[s];
    const int t0 = sp * SPLIT;
    if (t0 >= L) return;  // workgroup-uniform
    const int tid = threadIdx.x;
    const int cc = tid & 15;
    const int hr = (tid >> 4) % (HW < 16 ? HW : 16);
    const int tl = TL > 1 ? tid / PAIRS : 0;
    const int ntok = min(SPLIT, L - t0);
    const int page = min(max(page_table[(size_t)s * max_pages + t0 / kPage], 0), num_pages - 1);
    const int slot0 = t0 % kPage;
    const size_t tstride = (size_t)H * kD;  // elements between consecutive tokens
    size_t base[HPT];
    float q[HPT][8], m[HPT], l[HPT], o[HPT][8];
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
        const int h = hg * HW + hr + 16 * j;
        base[j] = (((size_t)page * kPage + slot0) * H + h) * kD + cc * 8;
        to_float8<T>(*(const s16x8 *)(Qp + ((size_t)s * H + h) * kD + cc * 8), q[j]);
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
    }

    s16x8 kx[2][HPT][B], vx[2][HPT][B];
    auto load = [&](int buf, int b) {
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int tt = (b * B + u) * TL + tl;
#pragma unroll
            for (int j = 0; j < HPT; ++j) {
                if (tt < ntok) {
                    kx[buf][j][u] = stream_load(Kp + base[j] + tt * tstride);
                    vx[buf][j][u] = stream_load(Vp + base[j] + tt * tstride);
                } else {
                    kx[buf][j][u] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
                    vx[buf][j][u] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
                }
            }
        }
    };
    auto consume = [&](int buf, int b) {
#pragma unroll
        for (int j = 0; j < HPT; ++j) {
            float sc[B];
            float mb = -INFINITY;
#pragma unroll
            for (int u = 0; u < B; ++u) {
                float kf[8];
                to_float8<T>(kx[buf][j][u], kf);
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) dot = fmaf(q[j][e], kf[e], dot);
                dot = row16_sum(dot);
                const int tt = (b * B + u) * TL + tl;
                sc[u] = tt < ntok ? dot * c : -INFINITY;
                mb = fmaxf(mb, sc[u]);
            }
            const float mn = fmaxf(m[j], mb);
            const float mu = (mn == -INFINITY) ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m[j] - mu);
            m[j] = mn;
            l[j] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[j][e] *= alpha;
#pragma unroll
            for (int u = 0; u < B; ++u) {
                const float p = __builtin_amdgcn_exp2f(sc[u] - mu);
                l[j] += p;
                float vf[8];
                to_float8<T>(vx[buf][j][u], vf);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[j][e] = fmaf(p, vf[e], o[j][e]);
            }
        }
    };

    load(0, 0);
    for (int b = 0; b < NB; b += 2) {
        load(1, b + 1);
        consume(0, b);
        if (b + 2 < NB) load(0, b + 2);
        consume(1, b + 1);
    }

    // Merge the token lanes through LDS (HW = 8 only), then write the split's partials.
    if constexpr (TL > 1) {
        __shared__ float xm[PAIRS], xl[PAIRS], xo[PAIRS * 9];
        if (tl == 1) {
            xm[tid - PAIRS] = m[0];
            xl[tid - PAIRS] = l[0];
#pragma unroll
            for (int e = 0; e < 8; ++e) xo[(tid - PAIRS) * 9 + e] = o[0][e];
        }
        __syncthreads();
        if (tl != 0) return;
        const float m1 = xm[tid], l1 = xl[tid];
        const float mn = fmaxf(m[0], m1);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float a0 = __builtin_amdgcn_exp2f(m[0] - mu), a1 = __builtin_amdgcn_exp2f(m1 - mu);
        l[0] = l[0] * a0 + l1 * a1;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[0][e] = o[0][e] * a0 + xo[tid * 9 + e] * a1;
        m[0] = mn;
    }
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
        const int h = hg * HW + hr + 16 * j;
        const float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;
        const size_t slot = ((size_t)s * H + h) * max_splits + sp;
        float *po = part_o + slot * kD + cc * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) po[e] = o[j][e] * inv;
        if (cc == 0) part_lse[slot] = l[j] > 0.f ? m[j] + __builtin_amdgcn_logf(l[j]) : -INFINITY;
    }
}

// Combine: grid (S, H), one wave per (sequence, head); lane i owns columns 2i and 2i+1.
// Partial lse values are in log2 units. The partial
// results of up to kCombineBatch splits are loaded together (one memory round trip per
// batch), and the merge keeps a running maximum of the partial lse values, rescaling the
// running sums when a later batch raises it, so no separate pass finds the maximum first.
constexpr int kCombineThreads = 64;
constexpr int kCombineBatch = 32;

template <typename T>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse,
    const int32_t *__restrict__ seq_lens, uint16_t *__restrict__ O, float *__restrict__ LSE,
    int H, int max_splits, int split)
{
    const int s = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
    const int ns = min((seq_lens[s] + split - 1) / split, max_splits);
    const size_t slot0 = ((size_t)s * H + h) * max_splits;

    float mu = -INFINITY, wsum = 0.f;  // running maximum (log2 units) and sum of weights
    float2 acc = {0.f, 0.f};
    for (int j0 = 0; j0 < ns; j0 += kCombineBatch) {
        float2 o[kCombineBatch];
        float lw[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const int j = j0 + u;
            o[u] = j < ns ? *(const float2 *)(part_o + (slot0 + j) * kD + 2 * i) : float2{0.f, 0.f};
            lw[u] = j < ns ? part_lse[slot0 + j] : -INFINITY;
        }
        float bm = lw[0];
#pragma unroll
        for (int u = 1; u < kCombineBatch; ++u) bm = fmaxf(bm, lw[u]);
        const float nm = fmaxf(mu, bm);
        if (nm == -INFINITY) continue;  // no split so far has a visible key
        const float r = __builtin_amdgcn_exp2f(mu - nm);  // 0 while mu is -inf
        acc.x *= r;
        acc.y *= r;
        wsum *= r;
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const float w = __builtin_amdgcn_exp2f(lw[u] - nm);
            acc.x = fmaf(w, o[u].x, acc.x);
            acc.y = fmaf(w, o[u].y, acc.y);
            wsum += w;
        }
        mu = nm;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    uint16_t *op = O + ((size_t)s * H + h) * kD + 2 * i;
    op[0] = from_float<T>(acc.x * inv);
    op[1] = from_float<T>(acc.y * inv);
    if (LSE != nullptr && i == 0)
        LSE[(size_t)s * H + h] = wsum > 0.f ? (mu + __builtin_amdgcn_logf(wsum)) * kLn2 : -INFINITY;
}

template <typename T, int HW, int SPLIT>
hipError_t launch_split(const DecodeArgs &a, hipStream_t st, int max_splits, float *part_o,
                        float *part_lse)
{
    hipLaunchKernelGGL((decode_split_kernel<T, HW, SPLIT>),
                       dim3((unsigned)(a.H / HW), (unsigned)max_splits, (unsigned)a.S),
                       dim3(kThreads), 0, st, (const uint16_t *)a.q, (const uint16_t *)a.k_pages,
                       (const uint16_t *)a.v_pages, a.page_table, a.seq_lens, part_o, part_lse,
                       a.H, a.max_pages, a.num_pages, max_splits, a.scale * kLog2e);
    return hipGetLastError();
}

int splits_for(const DecodeArgs &a, int split)
{
    return (int)(((long)a.max_pages * kPage + split - 1) / split);
}

template <typename T, int HW>
hipError_t launch_width(const DecodeArgs &a, hipStream_t st, int split, float *part_o,
                        float *part_lse)
{
    const int max_splits = splits_for(a, split);
    if (split == 256) return launch_split<T, HW, 256>(a, st, max_splits, part_o, part_lse);
    if (split == 128) return launch_split<T, HW, 128>(a, st, max_splits, part_o, part_lse);
    return launch_split<T, HW, 64>(a, st, max_splits, part_o, part_lse);
}

constexpr long kMinSplitGroups = 512;

// Split length the launch uses: the largest (fewer, longer streams and fewer partials;
// measured fastest on the 8 x 4096..8192-token workload) that still gives at least
// kMinSplitGroups workgroups when every sequence is as long as the page table allows.
int pick_split(const DecodeArgs &a)
{
    const int hw = a.H % 16 == 0 ? 16 : 8;
    for (int cand = 256; cand > 64; cand /= 2)
        if ((long)a.S * (a.H / hw) * (((long)a.max_pages * kPage) / cand) >= kMinSplitGroups)
            return cand;
    return 64;
}

template <typename T>
hipError_t launch(const DecodeArgs &a, hipStream_t st)
{
    const int hw = a.H % 16 == 0 ? 16 : 8;
    const int split = pick_split(a);
    const int max_splits = splits_for(a, split);
    // partial O [S, H, max_splits, d] then partial lse [S, H, max_splits], both fp32
    float *part_o = (float *)a.workspace;
    float *part_lse = part_o + (size_t)a.S * a.H * max_splits * kD;
    const hipError_t e = hw == 16 ? launch_width<T, 16>(a, st, split, part_o, part_lse)
                                  : launch_width<T, 8>(a, st, split, part_o, part_lse);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel<T>, dim3((unsigned)a.S, (unsigned)a.H),
                       dim3(kCombineThreads), 0, st, part_o, part_lse, a.seq_lens,
                       (uint16_t *)a.o, a.lse, a.H, max_splits, split);
    return hipGetLastError();
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

}  // namespace

// Scratch of the allocation-free decode entry point: the split partials live in this
// file-scope device array instead of a caller's workspace. Each GPU holds its own copy until
// the process ends; every call on a GPU reuses it (nothing needs clearing: the split pass
// writes every partial the combine pass reads).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

size_t decode_partials_bytes(const DecodeArgs &a)
{
    return (size_t)a.S * a.H * splits_for(a, pick_split(a)) * (kD + 1) * sizeof(float);
}

// Device address of `scratch` on the device `st` runs on (found once per device, with that
// device current; in host code the array's name is not a device address).
hipError_t decode_static_scratch(hipStream_t st, void **ptr)
{
    int dev = 0, cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (st != nullptr && (e = hipStreamGetDevice(st, &dev)) != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st)
{
    (void)hipGetLastError();
    return a.dtype == 1 ? launch<_Float16>(a, st) : launch<__bf16>(a, st);
}

}  // namespace teaf
