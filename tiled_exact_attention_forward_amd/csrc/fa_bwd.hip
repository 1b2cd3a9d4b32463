// fa_bwd.hip -- gradients of tiled exact attention (dQ, dK, dV) for gfx950 (MI355X).
//
// Method: the backward pass recomputes the score tiles instead of storing them (the pages
// stress that the N x N matrix never reaches HBM and that recomputation in the backward
// pass is cheap: ops-transformer article on zwxr.cn, section 2.2, and the ops-transformer
// article on gitcode.csdn.net, section 二.1). With the row statistics LSE saved by the
// forward pass, P = exp(S - LSE) is rebuilt tile by tile, and with D_i = dO_i . O_i
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),   dK = scale dS^T Q,   dQ = scale dS K.
//
// gfx950 mapping: two kernels, no atomics (results are deterministic).
//  * bwd_dq_kernel runs first: a workgroup owns 128 query rows (4 waves x 32) with Q and dO
//    in registers. Its prologue also reads O and forms the row statistics the gradient needs,
//    D_i = sum_c dO_ic O_ic and L_i = LSE_i log2 e (+inf for a row without a visible key, so
//    its P is 0), and stores them per 32-row tile so that one 256-byte load brings a tile's
//    statistics to the dK/dV kernel. It then walks the visible 32-key tiles like the forward
//    pass: S^T = K Q^T and dP^T = V dO^T with lanes indexed by row, then dQ^T += K^T dS^T.
//  * bwd_dkdv_kernel: a workgroup owns 256 keys (4 waves x 64) with their K and V rows in
//    registers and walks the 32-row query tiles that can see them. It computes S = Q K^T and
//    dP = dO V^T with lanes indexed by key, so that P and dS convert in place into the B
//    operand of dV^T += dO^T P and dK^T += Q^T dS; Q^T and dO^T come from LDS through
//    ds_read_b64_tr_b16.
// Tiles stream from HBM to LDS with buffer_load ... lds through 4-slot rings. Scores, P, dS
// and all accumulators are fp32; P and dS are rounded to the input type for the products.
#include "fa_device.h"

namespace teaf {
namespace {

// Q/dO tiles of 32 rows stream through a 4-slot ring (like the forward's K/V ring; the
// "K" half of the ring holds Q, the "V" half dO). Each slot also holds the tile's row
// statistics: 32 L values then 32 values of -D (256 bytes).
constexpr int kBwdStages = 4;
template <int D>
using CfgBD = CfgSP<D, kBwdStages, 4>;
constexpr int kStatsBytes = 256;

// Row statistics are stored per 32-row tile of each (b, h): [L_0..L_31, -D_0..-D_31], so one
// 256-byte load brings a tile's statistics (-D as the dK/dV kernel starts its dP accumulation
// from it). Rows past Nq hold L = +inf (P = 0) and D = 0.
__host__ __device__ inline size_t stats_index(size_t bh, int nt32, int row)
{
    return ((size_t)bh * nt32 + (size_t)(row >> 5)) * 64 + (size_t)(row & 31);
}

// Swizzle of the backward's LDS tiles, which are read both row-wise (16 consecutive rows at
// one 16-byte chunk per 16 lanes, ds_read_b128) and transposed (4 consecutive rows x 4
// consecutive chunks per 32 lanes, ds_read_b64_tr_b16). XOR with the row's two 2-bit fields
// swapped spreads both patterns over all 64 banks; the forward's K swizzle (XOR with the row's
// low bits) spreads only the first and leaves the second 4-way conflicted (2-way at d 64).
template <int D>
__device__ __forceinline__ int b_swz(int row, int chunk)
{
    return D == 128 ? chunk ^ (((row & 3) << 2) | ((row >> 2) & 3))
                    : chunk ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Byte offsets (relative to a tile) of the transposed 16-bit reads that hand each lane four
// consecutive rows of one column, for tiles stored with b_swz: half h covers rows
// 8h .. 8h+7 of each 16-row chunk (the swizzle depends on the row within 16, so the two
// halves need their own offsets; whole 16-row chunks add 16 rows).
template <int D>
__device__ __forceinline__ int tr_ofs(int lane, int h, int db)
{
    constexpr int ROWB = 2 * D;
    const int g = lane >> 5;
    const int trow = 8 * h + 4 * g + ((lane & 15) >> 2);
    const int tchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    return trow * ROWB + 16 * b_swz<D>(trow, 4 * db + tchunk) + 8 * (lane & 1);
}

// acc += a * b on the matrix cores with acc held in accumulation registers (AGPRs). The dK/dV
// kernel keeps 256 accumulator values per lane for a whole key block; pinning them to the
// AGPR file leaves the VGPRs to S and dP, which the compiler would otherwise move through
// the same AGPRs on every tile (this file is built so that the compiler's own MFMAs use
// VGPR destinations). The compiler does not see these as MFMAs, so the hazards it would
// handle are covered here: s_nop 2 gives at least the wait states a vector write of a or
// b needs before a matrix read of it, and the accumulators are read only after the
// kernel's loop ends with padding of its own.
template <typename T>
__device__ __forceinline__ void mma_agpr(f32x16 &acc, s16x8 a, s16x8 b)
{
    if constexpr (__is_same(T, __bf16))
        __asm__("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        __asm__("s_nop 2\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// 24 wait states after the last inline MFMA into acc[h][*] and before anything reads them:
// the accumulators are the statement's operands, which orders it after their writers and
// before their readers.
template <int NH, int NDB>
__device__ __forceinline__ void settle_agpr(f32x16 (&acc)[NH][NDB])
{
    static_assert(NDB == 2 || NDB == 4, "d 64 or 128");
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        if constexpr (NDB == 4)
            __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                             : "+a"(acc[h][0]), "+a"(acc[h][1]), "+a"(acc[h][2]), "+a"(acc[h][3]));
        else
            __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[h][0]), "+a"(acc[h][1]));
    }
}

// Rows that may see keys [k0, k1] (a superset; the element mask decides).
template <int MASK>
__device__ __forceinline__ void rows_seeing(int k0, int k1, int Nq, int Nkv, int W, int G, int &lo,
                                            int &hi)
{
    const int delta = Nkv - Nq;
    lo = 0;
    hi = Nq;
    if (MASK == 1) lo = k0 - delta;
    if (MASK == 2) {
        lo = k0 - delta;
        if (k0 >= G) hi = min(Nq, k1 + W - delta);  // ip - j < W for non-global keys
    }
    if (MASK == 3) {
        lo = k0 - W - delta;
        hi = min(Nq, k1 + W - delta + 1);
    }
    if (MASK == 4 && k0 >= G) lo = k0 - delta;
    lo = max(lo, 0);
}

// Visible rows of one key as a range of tile-row offsets: with the lane's rows at positions
// i0 + c (c = 8(e/4) + e%4, compile-time per element), key j is visible from row c when
// lo <= c <= hi. Equivalent to key_visible for masks 1-4.
template <int MASK>
__device__ __forceinline__ void key_row_range(int j, int i0, int W, int G, int &lo, int &hi)
{
    const int a = j - i0;  // c >= a  <=>  j <= i0 + c (causal)
    lo = a;
    hi = INT_MAX;
    if (MASK == 2 && j >= G) hi = a + W - 1;  // i - j < W
    if (MASK == 3) {
        lo = a - W;
        hi = a + W;
    }
    if (MASK == 4 && j < G) lo = INT_MIN;
}

// True when every key in [k0, k1] is visible from every position in [i0, i1].
template <int MASK>
__device__ __forceinline__ bool block_visible(int i0, int i1, int k0, int k1, int W, int G)
{
    if (MASK == 0) return true;
    if (MASK == 1) return k1 <= i0;
    if (MASK == 2) return k1 <= i0 && (i1 - k0 < W || k1 < G);
    if (MASK == 3) return k0 >= i1 - W && k1 <= i0 + W;
    return k1 <= i0 || k1 < G;
}

// One 32-row tile of the dK/dV kernel for this wave's 32 NH keys (NH halves of 32): qt, gt
// and st are the tile's
// Q, dO and statistics in LDS, vw the wave's V rows. The pointers are restrict-qualified:
// nothing else in the step touches that memory, which also tells the compiler that the
// loads of later tiles into other slots, still in flight, cannot overlap these reads.
template <typename T, typename C, int MASK, int NH>
__device__ __forceinline__ void dkdv_step(const char *__restrict__ qt, const char *__restrict__ gt,
                                          const char *__restrict__ vw,
                                          const float *__restrict__ st,
                                          const s16x8 (&kf)[NH][C::NKK],
                                          f32x16 (&dkt)[NH][C::NDB], f32x16 (&dvt)[NH][C::NDB],
                                          const int (&kofs)[C::NKK], const int (&tro)[2][C::NDB],
                                          float c, int ip0, int kw, int li, int g, int W, int G)
{
    using Op = Ops16<T>;
    constexpr int BN = 32, NKK = C::NKK, NDB = C::NDB;
    f32x16 s[2], dp[2];  // per half (only [0] when NH = 1)
    {
        // all Q fragments first, then both halves' MFMAs, which share each fragment
        s16x8 a[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) a[kk] = *(const s16x8 *)(qt + kofs[kk]);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            s[0] = Op::mma(a[kk], kf[0][kk], kk == 0 ? f32x16{} : s[0]);
            if constexpr (NH == 2) s[1] = Op::mma(a[kk], kf[1][kk], kk == 0 ? f32x16{} : s[1]);
        }
    }
    // Block sparse: the workgroup visits only query blocks that see its key block, whole;
    // the other masks decide per element.
    const bool full = MASK == kBlockSparse ||
                      block_visible<MASK>(ip0, ip0 + BN - 1, kw, kw + 32 * NH - 1, W, G);
    int lo[2] = {INT_MIN, INT_MIN}, hi[2] = {INT_MAX, INT_MAX};
    if (MASK != 0 && MASK != kBlockSparse && !full) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
            key_row_range<MASK>(kw + 32 * h + li, ip0 + 4 * g, W, G, lo[h], hi[h]);
    }
    // dP = dO V^T; P = 2^(c S - L) is formed alongside, two elements of each half per
    // step, so that one wave keeps its matrix and vector units busy together.
    {
        f32x4 lv[4], nd4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) lv[q] = *(const f32x4 *)(st + 8 * q + 4 * g);
        // -D of the rows this lane's accumulator elements belong to: the dP chains start
        // from it, so they end at dP - D
#pragma unroll
        for (int q = 0; q < 4; ++q) nd4[q] = *(const f32x4 *)(st + 32 + 8 * q + 4 * g);
        const f32x16 nd = __builtin_shufflevector(
            __builtin_shufflevector(nd4[0], nd4[1], 0, 1, 2, 3, 4, 5, 6, 7),
            __builtin_shufflevector(nd4[2], nd4[3], 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2, 3, 4, 5,
            6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        // V fragments of the halves (rows 32 h + key; v1 unused when NH = 1)
        s16x8 a = *(const s16x8 *)(gt + kofs[0]);
        s16x8 v0 = *(const s16x8 *)(vw + kofs[0]);
        s16x8 v1 = NH == 2 ? *(const s16x8 *)(vw + 32 * C::ROWB + kofs[0]) : v0;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int kn = (kk + 1) % NKK;
            const s16x8 an = *(const s16x8 *)(gt + kofs[kn]);
            const s16x8 v0n = *(const s16x8 *)(vw + kofs[kn]);
            const s16x8 v1n = NH == 2 ? *(const s16x8 *)(vw + 32 * C::ROWB + kofs[kn]) : v0n;
            dp[0] = Op::mma(a, v0, kk == 0 ? nd : dp[0]);
            if constexpr (NH == 2) dp[1] = Op::mma(a, v1, kk == 0 ? nd : dp[1]);
#pragma unroll
            for (int e = 16 * kk / NKK; e < 16 * (kk + 1) / NKK; ++e) {
                const int r = 8 * (e >> 2) + (e & 3);
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    const float p =
                        fast_exp2(__builtin_fmaf(s[h][e], c, -lv[e >> 2][e & 3]));
                    s[h][e] = (MASK == 0 || MASK == kBlockSparse || (r >= lo[h] && r <= hi[h]))
                                  ? p
                                  : 0.f;
                }
            }
            a = an;
            v0 = v0n;
            v1 = v1n;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // dV^T += dO^T P; dS = P (dP - D) is formed alongside.
    {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const int o8 = 8 * kc;
            s16x8 pf[2];
#pragma unroll
            for (int h = 0; h < NH; ++h)
                pf[h] = Op::pack8(s[h][o8], s[h][o8 + 1], s[h][o8 + 2], s[h][o8 + 3],
                                  s[h][o8 + 4], s[h][o8 + 5], s[h][o8 + 6], s[h][o8 + 7]);
            const char *p0 = gt + kc * 16 * C::ROWB;
            s16x4 tlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + tro[0][0]));
            s16x4 thi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + tro[1][0]));
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int dn = (db + 1) % NDB;
                const s16x4 lon = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + tro[0][dn]));
                const s16x4 hin = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + tro[1][dn]));
                const s16x8 ta = __builtin_shufflevector(tlo, thi, 0, 1, 2, 3, 4, 5, 6, 7);
                mma_agpr<T>(dvt[0][db], ta, pf[0]);
                if constexpr (NH == 2) mma_agpr<T>(dvt[1][db], ta, pf[1]);
#pragma unroll
                for (int e = o8 + 8 * db / NDB; e < o8 + 8 * (db + 1) / NDB; ++e)
#pragma unroll
                    for (int h = 0; h < NH; ++h)
                        dp[h][e] = s[h][e] * dp[h][e];
                tlo = lon;
                thi = hin;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // dK^T += Q^T dS
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const int o8 = 8 * kc;
        s16x8 sf[2];
#pragma unroll
        for (int h = 0; h < NH; ++h)
            sf[h] = Op::pack8(dp[h][o8], dp[h][o8 + 1], dp[h][o8 + 2], dp[h][o8 + 3],
                              dp[h][o8 + 4], dp[h][o8 + 5], dp[h][o8 + 6], dp[h][o8 + 7]);
        const char *p0 = qt + kc * 16 * C::ROWB;
        s16x4 tlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + tro[0][0]));
        s16x4 thi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + tro[1][0]));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int dn = (db + 1) % NDB;
            const s16x4 lon = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + tro[0][dn]));
            const s16x4 hin = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + tro[1][dn]));
            const s16x8 ta = __builtin_shufflevector(tlo, thi, 0, 1, 2, 3, 4, 5, 6, 7);
            mma_agpr<T>(dkt[0][db], ta, sf[0]);
            if constexpr (NH == 2) mma_agpr<T>(dkt[1][db], ta, sf[1]);
            tlo = lon;
            thi = hin;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// dK and dV. A workgroup owns 256 keys, 64 per wave in two 32-key halves (NH = 2). K fragments
// stay in registers and V rows in LDS (64 KB, loaded once; registers go to the dK/dV
// accumulators); each Q or dO fragment read from LDS feeds both halves, which halves the LDS
// reads per MFMA against 32 keys per wave. Under a block-sparse layout a workgroup owns one
// 128-key block, 32 keys per wave (NH = 1): with two blocks per workgroup, every query block
// that sees only one of them would cost the other's products too. Per 32-row tile:
//   S = Q K^T, dP = dO V^T           (lanes indexed by key: lane (g, key) holds rows
//                                     8(e/4) + 4g + e%4 of each half)
//   P = 2^(c S - L), dS = P (dP - D) (elementwise, fp32)
//   dV^T += dO^T P, dK^T += Q^T dS   (P, dS converted in place into B operands; dO^T and Q^T
//                                     read transposed from LDS)
// The MFMA order (S of both halves, then dP while the exponentials of P run, then dV while
// dS is formed, then dK) lets one wave per SIMD overlap its vector and matrix work.
template <int MASK>
constexpr int dkdv_halves() { return MASK == kBlockSparse ? 1 : 2; }

template <typename T, int D, int MASK>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ ST, uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int Nq,
    int Nkv, float c, float scale, int W, int G, int nkt, int nt32,
    const uint8_t *__restrict__ layout, int H)
{
    using C = CfgBD<D>;
    using Op = Ops16<T>;
    constexpr int BN = 32, NKK = C::NKK, NDB = C::NDB, NS = kBwdStages, LPW = C::LPW;
    constexpr int NH = dkdv_halves<MASK>();  // 32-key halves per wave
    constexpr int KPB = 128 * NH;            // keys per workgroup
    extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];
    char *const lds = (char *)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, li = lane & 31;
    // Causal, window + global and prefix LM: the first key blocks see the most rows (causal:
    // the rows from the block's first key on; the global or prefix keys: every row), so when
    // every XCD holds whole heads, it runs its heads' key blocks in order of kb (all first
    // blocks, then all second ones, ...), longest first, and the blocks of little work fill
    // the end. Other masks: (b, h) major, the key blocks of a head side by side.
    int bh, kb;
    {
        const int per = (int)gridDim.x / kXcds;
        if ((MASK == 1 || MASK == 2 || MASK == 4) && (int)gridDim.x % kXcds == 0 &&
            per % nkt == 0) {
            const int hx = per / nkt, x = (int)blockIdx.x % kXcds, idx = (int)blockIdx.x / kXcds;
            bh = x * hx + idx % hx;
            kb = idx / hx;
        } else {
            const int L = xcd_remap(blockIdx.x, gridDim.x);
            bh = L / nkt;
            kb = L % nkt;
        }
    }
    const int k0 = kb * KPB;
    const int kw = k0 + wave * 32 * NH;  // this wave's first key
    const size_t qbase = (size_t)bh * Nq * D, kvbase = (size_t)bh * Nkv * D;
    const int delta = Nkv - Nq;

    // K rows of this lane's two keys as MFMA fragments (keys past Nkv read as zeros).
    s16x8 kf[NH][NKK];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int key = kw + 32 * h + li;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            kf[h][kk] = key < Nkv
                            ? *(const s16x8 *)(K + kvbase + (size_t)key * D + 16 * kk + 8 * g)
                            : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    // V rows of this wave's 32 NH keys go to LDS (after the ring and the statistics) with the
    // same swizzle as the Q and dO tiles (they share the read offsets), each wave loading its
    // own rows, zero past Nkv.
    char *const vl = lds + C::LDS_BYTES + NS * kStatsBytes;
#if defined(__HIP_DEVICE_COMPILE__)
    {
        const int rows = min(max(Nkv - kw, 0), 32 * NH);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(V + kvbase + (size_t)min(kw, Nkv - 1) * D), (short)0,
            rows * C::ROWB, 0x00020000);
        constexpr int VLOADS = 32 * NH * C::ROWB / 1024;  // wave-wide 1 KB loads
#pragma unroll
        for (int u = 0; u < VLOADS; ++u) {
            const int r = u * C::ROWS_PER_LOAD + lane / C::CHUNKS;
            const unsigned vo = r * C::ROWB + 16 * b_swz<D>(r, lane % C::CHUNKS);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vr, (lds_void *)(vl + (wave * 32 * NH + u * C::ROWS_PER_LOAD) * C::ROWB), 16, vo,
                0, 0, 0);
        }
    }
#endif
    f32x16 dkt[NH][NDB], dvt[NH][NDB];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int db = 0; db < NDB; ++db) dkt[h][db] = dvt[h][db] = f32x16{};

    // Q and dO tiles go to LDS like the forward's K tiles, swizzled by b_swz (read row-wise
    // for S and dP, transposed for dK and dV).
    unsigned off[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
        const int i = wave + C::NW * u;
        const int r = (i % C::KL) * C::ROWS_PER_LOAD + lane / C::CHUNKS;
        off[u] = r * C::ROWB + 16 * b_swz<D>(r, lane % C::CHUNKS);
    }
    int kofs[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kofs[kk] = li * C::ROWB + 16 * b_swz<D>(li, 2 * kk + g);
    int tro[2][NDB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < NDB; ++db) tro[h][db] = tr_ofs<D>(lane, h, db);
    const char *const vw = vl + wave * 32 * NH * C::ROWB;  // this wave's V rows

    // The 32-row tiles this workgroup visits: a range of tiles for masks 0-4; for the
    // block-sparse layout, the query blocks that see its 128-key block, listed in LDS after
    // the V rows.
    constexpr int TPQ = kSparseBlock / BN;  // 32-row tiles per query block
    int t0 = 0, ntl = 0;
    char *const lst = vl + KPB * C::ROWB;
    const uint16_t *qlist = (const uint16_t *)(lst + 16);
    if constexpr (MASK == kBlockSparse) {
        const int nkb = (Nkv + kSparseBlock - 1) / kSparseBlock;
        const int nqb = (Nq + kSparseBlock - 1) / kSparseBlock;
        static_assert(KPB == kSparseBlock, "one key block per workgroup");
        const uint8_t *lh = layout + (size_t)(bh % H) * nqb * nkb + k0 / kSparseBlock;
        const int n = compact_list<C::NW>((int *)lst, (uint16_t *)qlist, nqb, tid,
                                          [&](int qb) { return lh[(size_t)qb * nkb] != 0; });
        if (n > 0) {
            const int last = __builtin_amdgcn_readfirstlane((int)qlist[n - 1]);
            ntl = TPQ * (n - 1) + (last == nqb - 1 ? nt32 - TPQ * last : TPQ);
        }
    } else {
        int rlo, rhi;
        rows_seeing<MASK>(k0, min(k0 + KPB - 1, Nkv - 1), Nq, Nkv, W, G, rlo, rhi);
        t0 = rlo / BN;
        ntl = rhi > rlo ? (rhi + BN - 1) / BN - t0 : 0;
    }
    // Tile n of the stream (n < ntl): its index among the 32-row tiles (block sparse: tile
    // n % TPQ of the listed query block n / TPQ).
    auto tile32 = [&](int n) {
        if constexpr (MASK == kBlockSparse)
            return __builtin_amdgcn_readfirstlane((int)qlist[n / TPQ] * TPQ + n % TPQ);
        else
            return t0 + n;
    };
    const char *qb = (const char *)(Q + qbase);
    const char *gb = (const char *)(dO + qbase);
    [[maybe_unused]] const float *stb = ST + (size_t)bh * nt32 * 64;  // device code only
    auto qslot = [&](int n) { return lds + (n % NS) * C::TILEB; };
    auto gslot = [&](int n) { return lds + C::VREG + (n % NS) * C::TILEB; };
    auto sslot = [&](int n) { return lds + C::LDS_BYTES + (n % NS) * kStatsBytes; };
    // Tile n of the stream (rows (t0 + n) * 32 ..): its Q and dO share of this wave, and the
    // tile's statistics (every wave loads the same 256 bytes to the same place, so each
    // wave's own wait covers them). Every step issues a load so that every wait has the same
    // count; past the last tile the loads have an empty range (they only write zeros into
    // the slot of a tile already consumed) and touch no memory.
    auto load = [&](int n) {
        const bool real = n < ntl;
        const int tn = MASK == kBlockSparse ? (real ? tile32(n) : 0) : t0 + n;
        const int row0 = real ? tn * BN : Nq;
        issue_kv<C>(qb, gb, off, row0, Nq, qslot(n), gslot(n), wave);
#if defined(__HIP_DEVICE_COMPILE__)
        const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(stb + (real ? (size_t)tn * 64 : 0)), (short)0,
            real ? kStatsBytes : 0, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void *)sslot(n), 4, lane * 4, 0, 0, 0);
#endif
    };
    constexpr int kAhead = (NS - 2) * (LPW + 1);  // loads of the tiles after the next one

#pragma unroll
    for (int j = 0; j < NS - 1; ++j) load(j);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAhead));  // tile 0, the K and V rows
    ring_barrier();

    auto step = [&](int n) {
        load(n + NS - 1);
        const char *qt = qslot(n), *gt = gslot(n);
        const float *st = (const float *)sslot(n);
        const int ip0 = tile32(n) * BN + delta;  // absolute position of the tile's row 0

        dkdv_step<T, C, MASK, NH>(qt, gt, vw, st, kf, dkt, dvt, kofs, tro, c, ip0, kw, li, g, W,
                                  G);
        // tile n + 1 resident (the NS - 2 tiles after it may still be in flight), then publish
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAhead));
        ring_barrier();
    };
    // unrolled by the ring depth, so the slot offsets are constants
    static_assert(NS == 4, "the main loop is unrolled by the ring depth");
    int n = 0;
    for (; n + 3 < ntl; n += 4) {
        step(n);
        step(n + 1);
        step(n + 2);
        step(n + 3);
    }
    for (; n < ntl; ++n) step(n);
    // Every wave's loads (the empty ones past the last tile included) have landed before any
    // wave reuses the ring for the output rows, and before the workgroup exits.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    // The last matrix results must be complete before vector reads of them (19 wait states
    // for a 16-pass MFMA; the inline MFMAs are invisible to the compiler's hazard checks).
    // The padding takes the accumulators as operands, so every MFMA that writes one comes
    // before it and every read of one after it, wherever the compiler places the reads.
    settle_agpr<NH, NDB>(dkt);
    settle_agpr<NH, NDB>(dvt);

    // dK^T / dV^T: lane (g, key) holds columns db*32 + 8(e/4) + 4g + e%4. Rows go out
    // through LDS (this wave's 64 rows, padded by 16 bytes against bank conflicts; the ring
    // is free after the last barrier) so that each store writes whole 256-byte rows: stores
    // of 16 bytes per row, all waves of the chip finishing together, left partly written
    // lines for the L2 to evict and write back more than once.
    constexpr int RP = C::ROWB + 16;
    static_assert(4 * 32 * NH * RP <= C::LDS_BYTES + NS * kStatsBytes + KPB * C::ROWB,
                  "staging");
    char *const stg = lds + wave * 32 * NH * RP;
#pragma unroll
    for (int t = 0; t < 2; ++t) {  // dK, then dV
        uint16_t *dst = (t == 0 ? dK : dV) + kvbase;
        const float f = t == 0 ? scale : 1.f;
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int blk = 0; blk < 4; ++blk) {
                    const f32x16 &acc = t == 0 ? dkt[h][db] : dvt[h][db];
                    *(s16x4 *)(stg + (32 * h + li) * RP + 2 * (db * 32 + 8 * blk + 4 * g)) =
                        Op::pack4(acc[4 * blk] * f, acc[4 * blk + 1] * f, acc[4 * blk + 2] * f,
                                  acc[4 * blk + 3] * f);
                }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done
        __asm__ volatile("" ::: "memory");
        constexpr int PER_ROW = C::ROWB / 16;  // 16-byte pieces of a row
#pragma unroll
        for (int it = 0; it < 32 * NH * PER_ROW / 64; ++it) {
            const int i = it * 64 + lane, r = i / PER_ROW, cpos = i % PER_ROW;
            const s16x8 val = *(const s16x8 *)(stg + r * RP + 16 * cpos);
            if (kw + r < Nkv) *(s16x8 *)(dst + (size_t)(kw + r) * D + 8 * cpos) = val;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next tensor's writes
        __asm__ volatile("" ::: "memory");
    }
}

// One 32-key tile of the dQ kernel: kt and vt are the tile's K and V in LDS
// (restrict-qualified: the loads of later tiles into other ring slots cannot overlap them).
// S^T = K Q^T and dP^T = V dO^T (lane (g, row) holds keys 8(e/4) + 4g + e%4), then
// dQ^T += K^T dS^T with K^T read transposed.
template <typename T, typename C, int MASK>
__device__ __forceinline__ void dq_step(const char *__restrict__ kt, const char *__restrict__ vt,
                                        const s16x8 (&qf)[C::NKK], const s16x8 (&gf)[C::NKK],
                                        f32x16 (&dqt)[C::NDB], const int (&kofs)[C::NKK],
                                        const int (&tro)[2][C::NDB], float c, float lrow,
                                        float drow, bool masked, int kv0, int ip, int Nkv, int W,
                                        int G, int g)
{
    using Op = Ops16<T>;
    constexpr int NKK = C::NKK, NDB = C::NDB;
    // the S and dP accumulation chains alternate, so no MFMA waits for its predecessor
    f32x16 s, dp;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        s = Op::mma(*(const s16x8 *)(kt + kofs[kk]), qf[kk], kk == 0 ? f32x16{} : s);
        dp = Op::mma(*(const s16x8 *)(vt + kofs[kk]), gf[kk], kk == 0 ? f32x16{} : dp);
    }
    if (masked) mask_tile<MASK>(s, kv0, ip, Nkv, W, G, g);
#pragma unroll
    for (int e = 0; e < 16; ++e) {  // hidden scores are -inf, c > 0: P = 2^-inf = 0
        const float p = fast_exp2(__builtin_fmaf(s[e], c, -lrow));
        dp[e] = p * (dp[e] - drow);
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const int o8 = 8 * kc;
        const s16x8 sf = Op::pack8(dp[o8], dp[o8 + 1], dp[o8 + 2], dp[o8 + 3], dp[o8 + 4],
                                   dp[o8 + 5], dp[o8 + 6], dp[o8 + 7]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int base = kc * 16 * C::ROWB;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(kt + base + tro[0][db]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(kt + base + tro[1][db]));
            dqt[db] = Op::mma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), sf,
                              dqt[db]);
        }
    }
}

// dQ. A workgroup owns 128 query rows (4 waves x 32) with Q and dO in registers and walks
// the visible 32-key tiles with the forward's schedule. K/V tiles stream through the
// forward's 4-slot ring; every step issues a load (empty past the last tile), so every wait
// has the same count.
constexpr int kDqStages = 4;
template <typename T, int D, int MASK>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const uint16_t *__restrict__ O, const float *__restrict__ LSE, float *__restrict__ ST,
    uint16_t *__restrict__ dQ, int Nq, int Nkv, float c, float scale, int W, int G, int nqt,
    int nt32, const uint8_t *__restrict__ layout, int H)
{
    using C = CfgSP<D, kDqStages, 4>;
    constexpr int SM = MASK == kBlockSparse ? 0 : MASK;  // element mask: the key tail only
    constexpr int BM = 128, BN = 32, NKK = C::NKK, NDB = C::NDB, NS = kDqStages, LPW = C::LPW;
    extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];
    char *const lds = (char *)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, li = lane & 31;
    const int Lb = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = Lb / nqt;
    const int q0 = (nqt - 1 - Lb % nqt) * BM;
    const int row = q0 + wave * 32 + li, ip = row + (Nkv - Nq);
    const size_t qbase = (size_t)bh * Nq * D, kvbase = (size_t)bh * Nkv * D;

    s16x8 qf[NKK], gf[NKK], of[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (row < Nq) {
            qf[kk] = *(const s16x8 *)(Q + qbase + (size_t)row * D + 16 * kk + 8 * g);
            gf[kk] = *(const s16x8 *)(dO + qbase + (size_t)row * D + 16 * kk + 8 * g);
            of[kk] = *(const s16x8 *)(O + qbase + (size_t)row * D + 16 * kk + 8 * g);
        } else {
            qf[kk] = gf[kk] = of[kk] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    // As in the forward, a negative scale moves into Q (sign bits flipped, exact; Q enters
    // only the scores here) and c is kept at least the smallest normal float, so a hidden
    // score (-inf) times c stays -inf and its P is 0 with no test.
    {
        const short qsign = c < 0.f ? (short)0x8000 : (short)0;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qf[kk] = qf[kk] ^ qsign;
        c = fmaxf(fabsf(c), 1.17549435e-38f);
    }
    // Row statistics: lanes i and i + 32 hold complementary halves of row i's columns.
    auto tof = [](short x) -> float {
        if constexpr (__is_same(T, __bf16))
            return __uint_as_float((unsigned)(unsigned short)x << 16);
        else
            return (float)__builtin_bit_cast(_Float16, x);
    };
    float dpart = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf(tof(gf[kk][e]), tof(of[kk][e]), dpart);
    const float drow = half_swap_sum(dpart);  // 0 for rows past Nq (zero fragments)
    float lrow = INFINITY;
    if (row < Nq) {
        const float lse = LSE[(size_t)bh * Nq + row];
        lrow = lse == -INFINITY ? INFINITY : lse * kLog2e;
    }
    // Stored for the dK/dV kernel, which runs next, for every row of the 32-row tiles (rows
    // past Nq hold L = +inf, so their P is 0, and D = 0).
    if (g == 0 && row < nt32 * 32) {
        ST[stats_index(bh, nt32, row)] = lrow;
        ST[stats_index(bh, nt32, row) + 32] = -drow;
    }

    const TileSchedule sch = make_schedule<SM, BM, BN>(q0, Nq, Nkv, W, G);
    int ntl = sch.total, nint = sch.interior;
    // Block sparse: the key blocks this query block sees, listed in LDS after the ring as in
    // the forward (key_block_list); only the key-tail tile is masked.
    constexpr int TPB = kSparseBlock / BN;
    const uint16_t *blist = (const uint16_t *)(lds + C::LDS_BYTES + 16);
    if constexpr (MASK == kBlockSparse) {
        const int nkb = (Nkv + kSparseBlock - 1) / kSparseBlock;
        const uint8_t *lrow = layout + ((size_t)(bh % H) * nqt + q0 / kSparseBlock) * nkb;
        key_block_list<C::NW, BN>(lds + C::LDS_BYTES, lrow, nkb, Nkv, tid, ntl, nint);
    }
    auto tile_at = [&](int p, const TileSchedule::Cursor &cu) {  // key tile at position p
        if constexpr (MASK == kBlockSparse)
            return __builtin_amdgcn_readfirstlane((int)blist[p / TPB] * TPB + p % TPB);
        else
            return cu.t;
    };
    f32x16 dqt[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqt[db] = f32x16{};

    unsigned off[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
        const int i = wave + C::NW * u;
        const int r = (i % C::KL) * C::ROWS_PER_LOAD + lane / C::CHUNKS;
        off[u] = r * C::ROWB + 16 * b_swz<D>(r, lane % C::CHUNKS);
    }
    int kofs[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kofs[kk] = li * C::ROWB + 16 * b_swz<D>(li, 2 * kk + g);
    int tro[2][NDB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < NDB; ++db) tro[h][db] = tr_ofs<D>(lane, h, db);

    const char *kb = (const char *)(K + kvbase);
    const char *vb = (const char *)(V + kvbase);
    auto kslot = [&](int n) { return lds + ((unsigned)n % NS) * C::TILEB; };
    auto vslot = [&](int n) { return lds + C::VREG + ((unsigned)n % NS) * C::TILEB; };
    // Tile n of the stream goes to slot n % NS; past the last tile the load is empty
    // (zero rows: it touches no memory and only writes zeros into a consumed slot).
    TileSchedule::Cursor ld = sch.begin(), cur = sch.begin();
    auto load = [&](int n) {
        const int kv0 = n < ntl ? tile_at(n, ld) * BN : Nkv;
        issue_kv<C>(kb, vb, off, kv0, Nkv, kslot(n), vslot(n), wave);
        if (n < ntl) ld = sch.next(ld);
    };
    constexpr int kAhead = (NS - 2) * LPW;  // loads of the tiles after the next one
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) load(j);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAhead));  // tile 0 (and the Q, dO rows)
    ring_barrier();
    // Steady state (like the forward's): tiles n .. n + 3 unmasked and their look-ahead loads
    // interior, so the tile index comes from the schedule position, the mask is compiled
    // out, and the loop is unrolled by the ring depth (slot offsets are constants).
    static_assert(NS == 4, "the steady loop is unrolled by the ring depth");
    auto steady = [&](int n) {
        const int p = n + NS - 1;
        const int tp = MASK == kBlockSparse ? tile_at(p, ld) : sch.interior_tile(p);
        issue_kv<C>(kb, vb, off, tp * BN, Nkv, kslot(p), vslot(p), wave);
        dq_step<T, C, SM>(kslot(n), vslot(n), qf, gf, dqt, kofs, tro, c, lrow, drow, false, 0,
                          ip, Nkv, W, G, g);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAhead));  // tile n + 1 resident
        ring_barrier();
    };
    int n = 0;
    for (; n + 3 + NS - 1 < nint; n += 4) {
        steady(n);
        steady(n + 1);
        steady(n + 2);
        steady(n + 3);
    }
    if (n > 0) {
        ld = sch.at(n + NS - 1);
        cur = sch.at(n);
    }
    for (; n < ntl; ++n) {
        load(n + NS - 1);
        dq_step<T, C, SM>(kslot(n), vslot(n), qf, gf, dqt, kofs, tro, c, lrow, drow, n >= nint,
                          tile_at(n, cur) * BN, ip, Nkv, W, G, g);
        cur = sch.next(cur);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAhead));  // tile n + 1 resident
        ring_barrier();
    }
    // dQ leaves as whole rows through the ring: every wave's loads (the empty ones past the
    // last tile included) must have landed and every wave must be done reading it.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    static_assert(4 * 32 * (C::ROWB + 16) <= C::LDS_BYTES, "dQ staging must fit the ring");
    store_rows_via_lds<T, D>(lds + wave * 32 * (C::ROWB + 16), dqt, scale, lane, dQ + qbase,
                             q0 + wave * 32, Nq, D);
}

template <typename T, int D, int MASK>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s)
{
    const int nt32 = (a.Nq + 31) / 32;
    float *st = (float *)a.workspace;
    const float c = a.scale * kLog2e;
    // dQ first: it also writes the row statistics the dK/dV kernel reads.
    using CB = CfgSP<D, kDqStages, 4>;
    const int nqt = (a.Nq + 127) / 128;
    // block sparse: wave counts and a list of up to kMaxKeyBlocks block ids after the ring
    constexpr int list_bytes = MASK == kBlockSparse ? 16 + 2 * kMaxKeyBlocks : 0;
    auto kb = bwd_dq_kernel<T, D, MASK>;
    const int lds_b = CB::LDS_BYTES + list_bytes;
    hipError_t e = hipFuncSetAttribute((const void *)kb,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_b);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kb, dim3((unsigned)((long)nqt * a.B * a.H)), dim3(256), lds_b, s,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       (const uint16_t *)a.dout, (const uint16_t *)a.o, a.lse, st,
                       (uint16_t *)a.dq, a.Nq, a.Nkv, c, a.scale, a.window, a.n_global, nqt, nt32,
                       a.layout, a.H);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    using CA = CfgBD<D>;
    constexpr int KPB = 128 * dkdv_halves<MASK>();  // keys per dK/dV workgroup
    const int nkt = (a.Nkv + KPB - 1) / KPB;
    const int lds_a = CA::LDS_BYTES + kBwdStages * kStatsBytes + KPB * CA::ROWB + list_bytes;
    auto ka = bwd_dkdv_kernel<T, D, MASK>;
    e = hipFuncSetAttribute((const void *)ka, hipFuncAttributeMaxDynamicSharedMemorySize, lds_a);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ka, dim3((unsigned)((long)nkt * a.B * a.H)), dim3(256), lds_a, s,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       (const uint16_t *)a.dout, st, (uint16_t *)a.dk, (uint16_t *)a.dv, a.Nq,
                       a.Nkv, c, a.scale, a.window, a.n_global, nkt, nt32, a.layout, a.H);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_mask(const BwdArgs &a, hipStream_t s)
{
    switch (a.mask) {
    case 0: return launch_bwd<T, D, 0>(a, s);
    case 1: return launch_bwd<T, D, 1>(a, s);
    case 2: return launch_bwd<T, D, 2>(a, s);
    case 3: return launch_bwd<T, D, 3>(a, s);
    case 4: return launch_bwd<T, D, 4>(a, s);
    default: return launch_bwd<T, D, kBlockSparse>(a, s);
    }
}

}  // namespace

hipError_t launch_backward(const BwdArgs &a, hipStream_t s)
{
    (void)hipGetLastError();
    if (a.dtype == 1)
        return a.d == 64 ? launch_bwd_mask<_Float16, 64>(a, s)
                         : launch_bwd_mask<_Float16, 128>(a, s);
    return a.d == 64 ? launch_bwd_mask<__bf16, 64>(a, s) : launch_bwd_mask<__bf16, 128>(a, s);
}

}  // namespace teaf
