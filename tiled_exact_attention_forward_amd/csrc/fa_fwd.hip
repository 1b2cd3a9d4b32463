// fa_fwd.hip -- tiled exact attention forward pass for gfx950 (MI355X, CDNA4).
//
// Method (ops-transformer article on gitcode.csdn.net, section 二.1 "FlashAttention算子";
// zwxr.cn article, section 3.1): a workgroup owns one tile of query rows, keeps them on
// chip, and walks the key/value tiles that its mask leaves visible. Per tile it forms the
// score block on the matrix cores, updates a running row maximum m and running sum l
// (online softmax), rescales the output accumulator by exp(m_old - m_new) and adds P V.
// After the last tile the accumulator is divided by l once. The N x N scores never leave
// registers. Scores, m, l and the accumulator are fp32 (the pages keep the softmax
// denominator in fp32); P is rounded to the input type for the P V product.
//
// gfx950 mapping (not the pages' Ascend tiling, which was sized for the 910's buffers):
//  * 256 threads = 4 wave64s, 128 query rows per workgroup, 32 rows per wave;
//    key/value tiles of 64 rows, double-buffered in LDS (prefetch of tile n+1 from HBM
//    into registers overlaps the math on tile n, then lands in the other LDS buffer).
//  * The score block is computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,
//    f16}: lane (g, i) then holds 16 keys of query row i per 32-key block, so the row max
//    and row sum are in-lane reductions plus one exchange with lane i^32, and the fp32
//    accumulator converts in place into the B operand (P^T) of O^T = V^T P^T.
//  * V stays row-major in LDS; the V^T operand is read with ds_read_b64_tr_b16, whose
//    16-lane transpose hands each lane four consecutive keys of one column.
//  * exp(x) is evaluated as 2^(x log2 e) with v_exp_f32; the log2 e factor is folded into
//    the score scale, so each score costs one multiply before the exponential.
//  * Tiles that a mask hides from every row are never loaded; tiles it hides from one
//    wave's rows skip that wave's math; only edge tiles evaluate the element mask.
//  * Workgroup ids are remapped so the query tiles of one (batch, head) run on one XCD and
//    share its L2 copy of K and V; the query tiles with the most visible keys go first.
//
// fp32 inputs use v_mfma_f32_32x32x2f32 (true fp32 products) in a simpler single-buffered
// kernel with 32-key tiles.
#include <limits.h>
#include <math.h>

#include "fa_launch.h"

namespace teaf {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;

// Hardware hands consecutive workgroup ids to the 8 XCDs in turn. Map id w (of n) to a
// logical index so that each XCD receives one contiguous run of logical indices.
__device__ __forceinline__ int xcd_remap(int w, int n)
{
    const int per = n / kXcds, rem = n % kXcds;
    const int x = w % kXcds, idx = w / kXcds;
    return (x < rem) ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

template <int MASK>
__device__ __forceinline__ bool key_visible(int ip, int j, int W, int G)
{
    if (MASK == 0) return true;
    if (MASK == 1) return j <= ip;
    return j <= ip && (ip - j < W || j < G);
}

// Key tiles visible to query rows [q0, min(q0+BM, Nq)): [a0,a1) then [b0,b1), ascending.
struct TileRanges {
    int a0, a1, b0, b1;
};

template <int MASK, int BM, int BN>
__device__ __forceinline__ TileRanges visible_tiles(int q0, int Nq, int Nkv, int W, int G)
{
    TileRanges r{0, (Nkv + BN - 1) / BN, 0, 0};
    if (MASK == 0) return r;
    const int delta = Nkv - Nq;
    const int last = min(Nkv - 1, min(q0 + BM, Nq) - 1 + delta);  // newest visible key
    if (last < 0) {
        r.a1 = 0;
        return r;
    }
    const int t_end = last / BN + 1;
    r.a1 = t_end;
    if (MASK == 1) return r;
    const int first = max(0, q0 + delta - W + 1);  // oldest window key of the first row
    const int w_begin = first / BN;
    const int g_end = (min(G, last + 1) + BN - 1) / BN;
    if (g_end >= w_begin) return r;  // global tiles touch the window: one range
    r.a1 = g_end;
    r.b0 = w_begin;
    r.b1 = t_end;
    return r;
}

// Key-tile schedule of one query tile: the visible tiles, ordered so that the tiles every
// row of the tile sees completely ("interior": no mask, no skip, no tail) come first and
// the remaining visible tiles ("edge") last: two interior ranges, then the visible parts of
// the two gaps the interior leaves (slots for every pairing of gap and visible range).
constexpr int kRanges = 6;
struct TileSchedule {
    int b[kRanges], e[kRanges];
    int interior, total;

    // Walks the schedule one tile at a time; work beyond an increment happens only when a
    // range ends.
    struct Cursor {
        int k, t, end;
    };
    __device__ __forceinline__ Cursor seek(int k) const
    {
        Cursor c{kRanges, 0, 0};
#pragma unroll
        for (int q = kRanges - 1; q >= 0; --q)
            if (q >= k && e[q] > b[q]) c = Cursor{q, b[q], e[q]};
        return c;
    }
    __device__ __forceinline__ Cursor begin() const { return seek(0); }
    __device__ __forceinline__ Cursor next(Cursor c) const
    {
        return c.t + 1 < c.end ? Cursor{c.k, c.t + 1, c.end} : seek(c.k + 1);
    }
};

__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

template <int MASK, int BM, int BN>
__device__ __forceinline__ TileSchedule make_schedule(int q0, int Nq, int Nkv, int W, int G)
{
    TileSchedule s;
#pragma unroll
    for (int k = 0; k < kRanges; ++k) s.b[k] = s.e[k] = 0;
    const TileRanges v = visible_tiles<MASK, BM, BN>(q0, Nq, Nkv, W, G);
    // interior ranges, judged for every row of the tile (padding rows included)
    const int delta = Nkv - Nq;
    const int ip0 = q0 + delta, ip1 = q0 + BM - 1 + delta;
    int lim = Nkv / BN;  // tiles without a key tail
    if (MASK >= 1) lim = min(lim, max(0, floor_div(ip0 + 1, BN)));  // causal for the first row
    int i0b = 0, i0e = lim, i1b = 0, i1e = 0;
    if (MASK == 2) {
        const int gend = G / BN;                                   // all keys global
        const int wbeg = max(0, -floor_div(-(ip1 - W + 1), BN));   // in every row's window
        i0e = min(gend, lim);
        i1b = max(wbeg, i0e);
        i1e = lim;
        if (i1b >= i1e) i1b = i1e = 0;
    }
    if (i0e <= i0b) i0b = i0e = 0;
    s.b[0] = i0b; s.e[0] = i0e;
    s.b[1] = i1b; s.e[1] = i1e;
    s.interior = (i0e - i0b) + (i1e - i1b);
    // edge ranges: the gaps between interior ranges, intersected with the visible ranges
    const int big = 0x3fffffff;
    const bool has1 = i1e > i1b;
    const int c0b = i0e, c0e = has1 ? i1b : big;   // gap after the first interior range
    const int c1b = has1 ? i1e : 0, c1e = has1 ? big : 0;  // gap after the second one
    auto put = [&s](int slot, int lo0, int hi0, int lo1, int hi1) {
        const int lo = max(lo0, lo1), hi = min(hi0, hi1);
        s.b[slot] = hi > lo ? lo : 0;
        s.e[slot] = hi > lo ? hi : 0;
    };
    put(2, c0b, c0e, v.a0, v.a1);
    put(3, c0b, c0e, v.b0, v.b1);
    put(4, c1b, c1e, v.a0, v.a1);
    put(5, c1b, c1e, v.b0, v.b1);
    s.total = 0;
#pragma unroll
    for (int q = 0; q < kRanges; ++q) s.total += s.e[q] - s.b[q];
    return s;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
struct Ops16;

template <>
struct Ops16<__bf16> {
    static __device__ __forceinline__ f32x16 mma(s16x8 a, s16x8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ s16x8 pack8(float a0, float a1, float a2, float a3,
                                                  float a4, float a5, float a6, float a7)
    {
        bf16x8 r = {(__bf16)a0, (__bf16)a1, (__bf16)a2, (__bf16)a3,
                    (__bf16)a4, (__bf16)a5, (__bf16)a6, (__bf16)a7};
        return __builtin_bit_cast(s16x8, r);
    }
    static __device__ __forceinline__ s16x4 pack4(float a0, float a1, float a2, float a3)
    {
        bf16x4 r = {(__bf16)a0, (__bf16)a1, (__bf16)a2, (__bf16)a3};
        return __builtin_bit_cast(s16x4, r);
    }
};

template <>
struct Ops16<_Float16> {
    static __device__ __forceinline__ f32x16 mma(s16x8 a, s16x8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ s16x8 pack8(float a0, float a1, float a2, float a3,
                                                  float a4, float a5, float a6, float a7)
    {
        f16x8 r = {(_Float16)a0, (_Float16)a1, (_Float16)a2, (_Float16)a3,
                   (_Float16)a4, (_Float16)a5, (_Float16)a6, (_Float16)a7};
        return __builtin_bit_cast(s16x8, r);
    }
    static __device__ __forceinline__ s16x4 pack4(float a0, float a1, float a2, float a3)
    {
        f16x4 r = {(_Float16)a0, (_Float16)a1, (_Float16)a2, (_Float16)a3};
        return __builtin_bit_cast(s16x4, r);
    }
};

// ------------------------------------------------------------------ 16-bit kernel

template <int D>
struct Cfg16 {
    static constexpr int BM = 128, BN = 64, NT = 256;
    static constexpr int ROWB = D * 2;                 // bytes of one K or V row
    static constexpr int TILEB = BN * ROWB;            // bytes of one K (or V) tile
    static constexpr int STAGEB = 2 * TILEB;           // K tile then V tile
    static constexpr int LDS_BYTES = 2 * STAGEB;       // two stages
    static constexpr int CHUNKS = ROWB / 16;           // 16-byte chunks per row
    static constexpr int ROWS_PER_LOAD = 64 / CHUNKS;  // rows one wave-wide 16-byte load fills
    static constexpr int LOADS = BN / ROWS_PER_LOAD / 4;  // loads per wave per tile and tensor
    static constexpr int NKK = D / 16, NDB = D / 32;
};

// LDS tiles are unpadded rows with an XOR swizzle of the 16-byte chunks (an involution:
// the same function maps logical to physical and back). Chosen against the 64-bank LDS:
// a ds_read_b128 serves 16 lanes per cycle, here 16 consecutive K rows at one logical
// chunk; a ds_read_b64_tr_b16 serves 32 lanes, here 4 consecutive V rows x 64 bytes.
template <int D>
__device__ __forceinline__ int k_swz(int row, int chunk)
{
    return D == 128 ? chunk ^ (row & 15) : chunk ^ ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row, int chunk)
{
    return D == 128 ? chunk ^ (4 * (row & 3)) : chunk ^ (4 * ((row >> 1) & 1));
}

typedef __attribute__((address_space(3))) void lds_void;

// Issue this wave's share of the direct HBM-to-LDS loads of the K and V tile that starts
// at key kv0 into the LDS stage `st`. Rows past Nkv read as zeros (buffer range check).
template <int D>
__device__ __forceinline__ void issue_tile(const char *kbh, const char *vbh,
                                           const unsigned (&koff)[Cfg16<D>::LOADS],
                                           const unsigned (&voff)[Cfg16<D>::LOADS], int kv0,
                                           int Nkv, char *st, int wave)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer resource type exists only for the GPU target
    using C = Cfg16<D>;
    kv0 = __builtin_amdgcn_readfirstlane(kv0);  // uniform: keeps the descriptors scalar
    // Raw buffer descriptors (gfx9 family word 3: data format 32, no swizzle; stride 0)
    // covering the keys from kv0 to the end: loads at or past that range return zeros.
    const int rest = (int)((unsigned)(Nkv - kv0) * C::ROWB);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(kbh + (size_t)kv0 * C::ROWB), (short)0, rest, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(vbh + (size_t)kv0 * C::ROWB), (short)0, rest, 0x00020000);
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
        const int slot = (4 * u + wave) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void *)(st + slot), 16, koff[u], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void *)(st + C::TILEB + slot), 16,
                                                 voff[u], 0, 0, 0);
    }
#endif
}

// The running maximum is only moved (and O, l rescaled) when a row's new maximum exceeds
// the one in use by more than this many powers of two; until then probabilities are taken
// relative to the stale maximum and stay below 2^8, which fp32 sums and 16-bit P hold
// exactly as well. The result is the same softmax: numerator and denominator share the
// reference value, and the final division removes it.
constexpr float kRescaleSlack = 8.0f;

// One 64-key tile for the 32 query rows of a wave. ks/vs: the tile's K and V in LDS.
// qf: Q^T fragments. c = scale * log2(e) >= 0 (a negative scale is folded into Q).
// MASKED tiles evaluate the element mask (and the key-range tail); others skip it.
template <typename T, int D, int MASK, bool MASKED>
__device__ __forceinline__ void attend_tile(const char *__restrict__ st,
                                            const int (&kofs)[D / 16], const int (&vofs)[D / 32],
                                            const s16x8 (&qf)[D / 16], f32x16 (&oacc)[D / 32],
                                            float &m, float &l, float c, int kv0, int ip,
                                            int Nkv, int W, int G, int lane)
{
    using C = Cfg16<D>;
    using Op = Ops16<T>;
    const int g = lane >> 5;
    const char *kb = st;
    const char *vb = st + C::TILEB;

    // S^T = K Q^T: A = K rows (keys) from LDS, B = Q^T fragments. Lane (g, j) reads row
    // 32jb + j, logical chunk 2kk + g.
    f32x16 sacc[2];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const s16x8 a = *(const s16x8 *)(kb + kofs[kk] + jb * 32 * C::ROWB);
            sacc[jb] = Op::mma(a, qf[kk], kk == 0 ? f32x16{} : sacc[jb]);
        }
    }

    // Lane (g, i) holds key 32jb + 8(e/4) + 4g + e%4 of row i in sacc[jb][e].
    float mx = -INFINITY;
    if constexpr (MASKED) {
        // The visible keys of a row form the range [lo, hi] plus the global keys [0, G);
        // offsets r = key - kv0 - 4g are compile-time constants per element. Scale first
        // (masked scores become -inf in the scaled domain), then mask.
        const int base = kv0 + 4 * g;
        const int hiR = (MASK == 0 ? Nkv - 1 : min(ip, Nkv - 1)) - base;
        const int loR = (MASK == 2 ? ip - W + 1 : INT_MIN / 2) - base;
        const int gR = (MASK == 2 ? G : 0) - base;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = jb * 32 + 8 * (e >> 2) + (e & 3);
                const bool vis = r <= hiR && (MASK != 2 || r >= loR || r < gR);
                sacc[jb][e] = vis ? sacc[jb][e] * c : -INFINITY;
                mx = fmaxf(mx, sacc[jb][e]);
            }
    } else {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[jb][e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = MASKED ? mx : mx * c;  // tile maximum of the scaled scores

    if (!__all(mt <= m + kRescaleSlack)) {
        const float mn = fmaxf(m, mt);
        const float alpha = fast_exp2(m - (mn == -INFINITY ? 0.f : mn));
        m = mn;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;

    float ps = 0.f;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float p = MASKED ? fast_exp2(sacc[jb][e] - mu)
                                   : fast_exp2(__builtin_fmaf(sacc[jb][e], c, -mu));
            sacc[jb][e] = p;
            ps += p;
        }
    l += ps;

    // O^T += V^T P^T over four 16-key chunks. Chunk kc, slot (g, e) is key
    // 16kc + 8(e/4) + 4g + e%4: P^T is sacc[kc/2][8(kc%2) + e] in place. The V^T operand
    // comes from two transposed reads of four keys each.
    // Lane (g, s, j) of a transposed read addresses row 16kc + 8h + 4g + j/4 and the
    // 8 bytes at element 32db + 16s + 4(j%4) (offset vofs[db] for kc = h = 0).
#pragma unroll
    for (int kc = 0; kc < C::BN / 16; ++kc) {
        const int jb = kc >> 1, o8 = 8 * (kc & 1);
        const s16x8 pf = Op::pack8(sacc[jb][o8 + 0], sacc[jb][o8 + 1], sacc[jb][o8 + 2],
                                   sacc[jb][o8 + 3], sacc[jb][o8 + 4], sacc[jb][o8 + 5],
                                   sacc[jb][o8 + 6], sacc[jb][o8 + 7]);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const char *p0 = vb + vofs[db] + kc * 16 * C::ROWB;
            const char *p1 = p0 + 8 * C::ROWB;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
            const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = Op::mma(a, pf, oacc[db]);
        }
    }
}

template <typename T, int D, int MASK>
__global__ __launch_bounds__(256, 2) void fwd16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE, int Nq,
    int Nkv, float c, int W, int G, int nqt)
{
    using C = Cfg16<D>;
    using Op = Ops16<T>;
    constexpr int BM = C::BM, BN = C::BN;
    extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, li = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nqt;
    const int q0 = (nqt - 1 - L % nqt) * BM;  // most-loaded query tiles first
    const int delta = Nkv - Nq;
    const size_t qbase = (size_t)bh * Nq * D, kvbase = (size_t)bh * Nkv * D;

    // Q^T fragments (B operand): lane (g, i) holds Q[row i][16kk + 8g .. +7]. A negative
    // scale is moved into Q by flipping sign bits (exact), so that c >= 0 below.
    const int wrow0 = q0 + wave * 32;
    const int row = wrow0 + li;
    const int ip = row + delta;
    const short qsign = c < 0.f ? (short)0x8000 : (short)0;
    c = fabsf(c);
    s16x8 qf[C::NKK];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
        if (row < Nq)
            qf[kk] = *(const s16x8 *)(Q + qbase + (size_t)row * D + 16 * kk + 8 * g) ^ qsign;
        else
            qf[kk] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }

    const TileSchedule sch = make_schedule<MASK, BM, BN>(q0, Nq, Nkv, W, G);

    float m = -INFINITY, l = 0.f;
    f32x16 oacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x16{};

    // K/V tiles go straight from HBM to LDS (buffer_load ... lds): wave-wide load u of
    // wave w fills the ROWS_PER_LOAD rows of slot q = 4u + w; lane l lands in physical
    // chunk l % CHUNKS of row q * ROWS_PER_LOAD + l / CHUNKS, so it fetches the logical
    // chunk the swizzle stores there. Offsets are relative to the tile's first key.
    const char *kbh = (const char *)(K + kvbase);
    const char *vbh = (const char *)(V + kvbase);
    unsigned koff[C::LOADS], voff[C::LOADS];
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
        const int r = (4 * u + wave) * C::ROWS_PER_LOAD + lane / C::CHUNKS;
        const int pc = lane % C::CHUNKS;
        koff[u] = r * C::ROWB + 16 * k_swz<D>(r, pc);
        voff[u] = r * C::ROWB + 16 * v_swz<D>(r, pc);
    }
    // Lane-constant LDS byte offsets of the swizzled operand reads (see attend_tile).
    int kofs[C::NKK], vofs[C::NDB];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) kofs[kk] = li * C::ROWB + 16 * k_swz<D>(li, 2 * kk + g);
    {
        const int trow = 4 * g + ((lane & 15) >> 2);
        const int tchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
            vofs[db] = trow * C::ROWB + 16 * v_swz<D>(trow, 4 * db + tchunk) + 8 * (lane & 1);
    }

    const int ntiles = sch.total;
    char *const lds = (char *)smem;
    TileSchedule::Cursor cur = sch.begin(), nxt = sch.next(cur);
    if (ntiles > 0) {
        issue_tile<D>(kbh, vbh, koff, voff, cur.t * BN, Nkv, lds, wave);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    // Interior tiles: every row sees every key, no per-wave decisions.
    for (int n = 0; n < sch.interior; ++n) {
        const int kv0 = cur.t * BN;
        if (n + 1 < ntiles)
            issue_tile<D>(kbh, vbh, koff, voff, nxt.t * BN, Nkv, lds + ((n + 1) & 1) * C::STAGEB,
                          wave);
        attend_tile<T, D, MASK, false>(lds + (n & 1) * C::STAGEB, kofs, vofs, qf, oacc, m, l, c,
                                       kv0, ip, Nkv, W, G, lane);
        cur = nxt;
        nxt = sch.next(nxt);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next tile have landed
        __syncthreads();
    }
    // Edge tiles: per wave, skip the tile, take it whole, or apply the element mask.
    for (int n = sch.interior; n < ntiles; ++n) {
        const int kv0 = cur.t * BN;
        if (n + 1 < ntiles)
            issue_tile<D>(kbh, vbh, koff, voff, nxt.t * BN, Nkv, lds + ((n + 1) & 1) * C::STAGEB,
                          wave);
        bool skip = wrow0 >= Nq;
        bool need_mask = kv0 + BN > Nkv;
        if (MASK >= 1) {
            const int ip0 = wrow0 + delta, ip1 = wrow0 + 31 + delta;
            if (kv0 > ip1) skip = true;
            if (kv0 + BN - 1 > ip0) need_mask = true;
            if (MASK == 2) {
                if (kv0 + BN - 1 < ip0 - W + 1 && kv0 >= G) skip = true;
                if (!(ip1 - kv0 < W) && !(kv0 + BN - 1 < G)) need_mask = true;
            }
        }
        const char *st = lds + (n & 1) * C::STAGEB;
        if (MASK == 0) {
            // without a mask the only edge tile is the key tail
            if (!skip)
                attend_tile<T, D, MASK, true>(st, kofs, vofs, qf, oacc, m, l, c, kv0, ip, Nkv, W,
                                              G, lane);
        } else if (!skip) {
            if (need_mask)
                attend_tile<T, D, MASK, true>(st, kofs, vofs, qf, oacc, m, l, c, kv0, ip, Nkv, W,
                                              G, lane);
            else
                attend_tile<T, D, MASK, false>(st, kofs, vofs, qf, oacc, m, l, c, kv0, ip, Nkv, W,
                                               G, lane);
        }
        cur = nxt;
        nxt = sch.next(nxt);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // Epilogue: both lane halves hold partial sums of the same row (same reference max).
    const float lt = l + __shfl_xor(l, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row < Nq) {
        uint16_t *orow = O + qbase + (size_t)row * D;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const s16x4 v4 = Op::pack4(oacc[db][4 * blk + 0] * inv, oacc[db][4 * blk + 1] * inv,
                                           oacc[db][4 * blk + 2] * inv, oacc[db][4 * blk + 3] * inv);
                *(s16x4 *)(orow + db * 32 + 8 * blk + 4 * g) = v4;
            }
        }
        if (g == 0)
            LSE[(size_t)bh * Nq + row] =
                lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    }
}

// ------------------------------------------------------------------ fp32 kernel

template <int D, int MASK>
__global__ __launch_bounds__(256) void fwd32_kernel(const float *__restrict__ Q,
                                                    const float *__restrict__ K,
                                                    const float *__restrict__ V,
                                                    float *__restrict__ O, float *__restrict__ LSE,
                                                    int Nq, int Nkv, float c, int W, int G, int nqt)
{
    constexpr int BM = 128, BN = 32, NT = 256, KP = D + 1;
    constexpr int NKK = D / 2, NDB = D / 32, RC = D / 4, CPT = BN * RC / NT;
    __shared__ float ks[BN * KP];
    __shared__ __attribute__((aligned(16))) float vs[BN * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, li = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nqt;
    const int q0 = (nqt - 1 - L % nqt) * BM;
    const int delta = Nkv - Nq;
    const size_t qbase = (size_t)bh * Nq * D, kvbase = (size_t)bh * Nkv * D;
    const int wrow0 = q0 + wave * 32, row = wrow0 + li, ip = row + delta;

    // Q^T fragments for the 32x32x2 MFMA: lane (g, i) holds Q[row i][2kk + g].
    float qf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = row < Nq ? Q[qbase + (size_t)row * D + 2 * kk + g] : 0.f;

    const TileRanges tr = visible_tiles<MASK, BM, BN>(q0, Nq, Nkv, W, G);
    const int na = tr.a1 - tr.a0, ntiles = na + (tr.b1 - tr.b0);
    float m = -INFINITY, l = 0.f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;

    for (int n = 0; n < ntiles; ++n) {
        const int tile = n < na ? tr.a0 + n : tr.b0 + (n - na);
        const int kv0 = tile * BN;
        __syncthreads();  // previous tile's readers are done
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int id = tid + u * NT, r = id / RC, cc = id % RC, key = kv0 + r;
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (key < Nkv) {
                kv = *(const f32x4 *)(K + kvbase + (size_t)key * D + 4 * cc);
                vv = *(const f32x4 *)(V + kvbase + (size_t)key * D + 4 * cc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ks[r * KP + 4 * cc + e] = kv[e];
            *(f32x4 *)(vs + r * D + 4 * cc) = vv;
        }
        __syncthreads();

        bool skip = wrow0 >= Nq;
        bool need_mask = kv0 + BN > Nkv;
        if (MASK >= 1) {
            const int ip0 = wrow0 + delta, ip1 = wrow0 + 31 + delta;
            if (kv0 > ip1) skip = true;
            if (kv0 + BN - 1 > ip0) need_mask = true;
            if (MASK == 2) {
                if (kv0 + BN - 1 < ip0 - W + 1 && kv0 >= G) skip = true;
                if (!(ip1 - kv0 < W) && !(kv0 + BN - 1 < G)) need_mask = true;
            }
        }
        if (skip) continue;

        f32x16 sacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[li * KP + 2 * kk + g], qf[kk], sacc, 0, 0, 0);
        float mt = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float t = sacc[e] * c;
            if (need_mask) {
                const int key = kv0 + 8 * (e >> 2) + 4 * g + (e & 3);
                if (key >= Nkv || !key_visible<MASK>(ip, key, W, G)) t = -INFINITY;
            }
            sacc[e] = t;
            mt = fmaxf(mt, t);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m, mt);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = fast_exp2(m - mu);
        m = mn;
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float p = fast_exp2(sacc[e] - mu);
            sacc[e] = p;
            ps += p;
        }
        l = l * alpha + ps;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
        // O^T += V^T P^T, one key per lane half per step: key 8blk + 4g + r.
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + 4 * g + (e & 3);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * D + db * 32 + li], sacc[e],
                                                                oacc[db], 0, 0, 0);
        }
    }

    const float lt = l + __shfl_xor(l, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row < Nq) {
        float *orow = O + qbase + (size_t)row * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                f32x4 v4 = {oacc[db][4 * blk] * inv, oacc[db][4 * blk + 1] * inv,
                            oacc[db][4 * blk + 2] * inv, oacc[db][4 * blk + 3] * inv};
                *(f32x4 *)(orow + db * 32 + 8 * blk + 4 * g) = v4;
            }
        if (g == 0)
            LSE[(size_t)bh * Nq + row] =
                lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    }
}

template <typename T, int D, int MASK>
hipError_t launch16(const FwdArgs &a, hipStream_t s)
{
    using C = Cfg16<D>;
    const int nqt = (a.Nq + C::BM - 1) / C::BM;
    const long nblk = (long)nqt * a.B * a.H;
    auto kern = fwd16_kernel<T, D, MASK>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(C::NT), C::LDS_BYTES, s,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       (uint16_t *)a.o, a.lse, a.Nq, a.Nkv, a.scale * kLog2e, a.window,
                       a.n_global, nqt);
    return hipGetLastError();
}

template <int D, int MASK>
hipError_t launch32(const FwdArgs &a, hipStream_t s)
{
    const int nqt = (a.Nq + 127) / 128;
    const long nblk = (long)nqt * a.B * a.H;
    hipLaunchKernelGGL((fwd32_kernel<D, MASK>), dim3((unsigned)nblk), dim3(256), 0, s,
                       (const float *)a.q, (const float *)a.k, (const float *)a.v, (float *)a.o,
                       a.lse, a.Nq, a.Nkv, a.scale * kLog2e, a.window, a.n_global, nqt);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch16_mask(const FwdArgs &a, hipStream_t s)
{
    switch (a.mask) {
    case 0: return launch16<T, D, 0>(a, s);
    case 1: return launch16<T, D, 1>(a, s);
    default: return launch16<T, D, 2>(a, s);
    }
}

template <int D>
hipError_t launch32_mask(const FwdArgs &a, hipStream_t s)
{
    switch (a.mask) {
    case 0: return launch32<D, 0>(a, s);
    case 1: return launch32<D, 1>(a, s);
    default: return launch32<D, 2>(a, s);
    }
}

}  // namespace

hipError_t launch_forward(const FwdArgs &a, hipStream_t s)
{
    (void)hipGetLastError();  // start from a clean error state
    if (a.dtype == 0) return a.d == 64 ? launch32_mask<64>(a, s) : launch32_mask<128>(a, s);
    if (a.dtype == 1)
        return a.d == 64 ? launch16_mask<_Float16, 64>(a, s) : launch16_mask<_Float16, 128>(a, s);
    return a.d == 64 ? launch16_mask<__bf16, 64>(a, s) : launch16_mask<__bf16, 128>(a, s);
}

}  // namespace teaf
