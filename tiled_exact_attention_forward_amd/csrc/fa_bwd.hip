// fa_bwd.hip -- gradients of tiled exact attention (dQ, dK, dV) for gfx950 (MI355X).
//
// Method: the backward pass recomputes the score tiles instead of storing them (the pages
// stress that the N x N matrix never reaches HBM and that recomputation in the backward
// pass is cheap: ops-transformer article on zwxr.cn, section 2.2, and the ops-transformer
// article on gitcode.csdn.net, section 二.1). With the row statistics LSE saved by the
// forward pass, P = exp(S - LSE) is rebuilt tile by tile, and with D_i = dO_i . O_i
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),   dK = scale dS^T Q,   dQ = scale dS K.
//
// gfx950 mapping: three kernels, no atomics (results are deterministic).
//  * bwd_rowdot_kernel: D_i = sum_c dO_ic O_ic and the log2-domain row statistic
//    L_i = LSE_i log2 e (+inf for a row without a visible key, so its P is 0).
//  * bwd_dkdv_kernel: a workgroup owns 128 keys (4 waves x 32) with their K and V rows in
//    registers and walks the 32-row query tiles that can see them. It computes S = Q K^T and
//    dP = dO V^T with lanes indexed by key, so that P and dS convert in place into the B
//    operand of dV^T += dO^T P and dK^T += Q^T dS; Q^T and dO^T come from LDS through
//    ds_read_b64_tr_b16.
//  * bwd_dq_kernel: a workgroup owns 128 query rows (4 waves x 32) with Q and dO in
//    registers and walks the visible 32-key tiles like the forward pass: S^T = K Q^T and
//    dP^T = V dO^T with lanes indexed by row, then dQ^T += K^T dS^T.
// Tiles stream from HBM to LDS with buffer_load ... lds into two stages. Scores, P, dS and
// all accumulators are fp32; P and dS are rounded to the input type for the products.
#include "fa_device.h"

namespace teaf {
namespace {

// Two-stage tiles of 32 rows, 4 waves: the same layout arithmetic as the forward's ring.
template <int D>
using CfgBD = CfgSP<D, 2, 4>;

// D_i and L_i for every row: 16 lanes per row, 8 elements each for d = 128 (4 for d = 64).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const uint16_t *__restrict__ O,
                                                         const uint16_t *__restrict__ dO,
                                                         const float *__restrict__ LSE,
                                                         float *__restrict__ Drow,
                                                         float *__restrict__ Lrow, long rows)
{
    constexpr int PER = D / 16;
    const long r = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int part = threadIdx.x & 15;
    float acc = 0.f;
    if (r < rows) {
        const uint16_t *o = O + r * D + part * PER;
        const uint16_t *g = dO + r * D + part * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const T a = __builtin_bit_cast(T, o[e]);
            const T b = __builtin_bit_cast(T, g[e]);
            acc = __builtin_fmaf((float)a, (float)b, acc);
        }
    }
    // sum over the 16 lanes of a row (DPP-free butterfly through lane shuffles)
#pragma unroll
    for (int s = 8; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 16);
    if (r < rows && part == 0) {
        Drow[r] = acc;
        const float lse = LSE[r];
        Lrow[r] = lse == -INFINITY ? INFINITY : lse * kLog2e;
    }
}

// Byte offsets (relative to a tile) of the transposed 16-bit reads that hand each lane four
// consecutive rows of one column, for tiles stored with the K swizzle: half h covers rows
// 8h .. 8h+7 of each 16-row chunk (the swizzle depends on the row within 16, so the two
// halves need their own offsets; whole 16-row chunks add 16 rows).
template <int D>
__device__ __forceinline__ int tr_ofs(int lane, int h, int db)
{
    constexpr int ROWB = 2 * D;
    const int g = lane >> 5;
    const int trow = 8 * h + 4 * g + ((lane & 15) >> 2);
    const int tchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    return trow * ROWB + 16 * k_swz<D>(trow, 4 * db + tchunk) + 8 * (lane & 1);
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

template <typename T, int D, int MASK>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ Drow, const float *__restrict__ Lrow, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, int Nq, int Nkv, float c, float scale, int W, int G, int nkt)
{
    using C = CfgBD<D>;
    using Op = Ops16<T>;
    constexpr int BN = 32, NKK = C::NKK, NDB = C::NDB;
    constexpr int STATS = C::LDS_BYTES;  // per stage: 32 L values then 32 D values
    extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];
    char *const lds = (char *)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, li = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nkt;
    const int k0 = (L % nkt) * 128;
    const int key = k0 + wave * 32 + li;
    const size_t qbase = (size_t)bh * Nq * D, kvbase = (size_t)bh * Nkv * D;

    // K and V rows of this lane's key as MFMA fragments (keys past Nkv read as zeros).
    s16x8 kf[NKK], vf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (key < Nkv) {
            kf[kk] = *(const s16x8 *)(K + kvbase + (size_t)key * D + 16 * kk + 8 * g);
            vf[kk] = *(const s16x8 *)(V + kvbase + (size_t)key * D + 16 * kk + 8 * g);
        } else {
            kf[kk] = vf[kk] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dkt[db] = dvt[db] = f32x16{};

    // Q and dO tiles (32 rows) go to LDS like the forward's K and V tiles, both with the K
    // swizzle (read row-wise for S and dP, transposed for dK and dV).
    unsigned off[C::LPW];
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
        const int i = wave + C::NW * u;
        const int r = (i % C::KL) * C::ROWS_PER_LOAD + lane / C::CHUNKS;
        off[u] = r * C::ROWB + 16 * k_swz<D>(r, lane % C::CHUNKS);
    }
    int kofs[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kofs[kk] = li * C::ROWB + 16 * k_swz<D>(li, 2 * kk + g);
    int tro[2][NDB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < NDB; ++db) tro[h][db] = tr_ofs<D>(lane, h, db);

    int rlo, rhi;
    rows_seeing<MASK>(k0, min(k0 + 127, Nkv - 1), Nq, Nkv, W, G, rlo, rhi);
    const int t0 = rlo / BN, t1 = rhi > rlo ? (rhi + BN - 1) / BN : t0;
    const char *qb = (const char *)(Q + qbase);
    const char *gb = (const char *)(dO + qbase);
    auto qslot = [&](int n) { return lds + (n & 1) * C::TILEB; };
    auto gslot = [&](int n) { return lds + C::VREG + (n & 1) * C::TILEB; };
    auto sslot = [&](int n) { return (float *)(lds + STATS + (n & 1) * 256); };
    // Statistics of the next tile travel through registers (loaded at the start of a step,
    // written to LDS at its end) so that no wait for them sits in the step.
    float nl = 0.f, nd = 0.f;
    auto load_stats = [&](int t) {
        const int row = t * BN + (lane & 31);
        nl = 0.f;
        nd = 0.f;
        if (wave == 0 && row < Nq) {  // rows past Nq: L = 0, D = 0 (their dO is zero)
            nl = Lrow[(size_t)bh * Nq + row];
            nd = Drow[(size_t)bh * Nq + row];
        }
    };
    auto store_stats = [&](int n) {
        if (wave == 0 && lane < 32) {
            sslot(n)[lane] = nl;
            sslot(n)[32 + lane] = nd;
        }
    };

    if (t1 > t0) {
        issue_kv<C>(qb, gb, off, t0 * BN, Nq, qslot(0), gslot(0), wave);
        load_stats(t0);
        __builtin_amdgcn_s_waitcnt(0);
        store_stats(0);
        __syncthreads();
    }
    for (int t = t0, n = 0; t < t1; ++t, ++n) {
        if (t + 1 < t1) {
            issue_kv<C>(qb, gb, off, (t + 1) * BN, Nq, qslot(n + 1), gslot(n + 1), wave);
            load_stats(t + 1);
        }
        const char *qt = qslot(n), *gt = gslot(n);
        const float *st = sslot(n);
        // S = Q K^T and dP = dO V^T: lane (g, key) holds rows 8(e/4) + 4g + e%4.
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            s = Op::mma(*(const s16x8 *)(qt + kofs[kk]), kf[kk], s);
            dp = Op::mma(*(const s16x8 *)(gt + kofs[kk]), vf[kk], dp);
        }
        f32x4 lv[4], dv4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            lv[q] = *(const f32x4 *)(st + 8 * q + 4 * g);
            dv4[q] = *(const f32x4 *)(st + 32 + 8 * q + 4 * g);
        }
        const int row0 = t * BN + (Nkv - Nq);  // absolute position of tile row 0
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = 8 * (e >> 2) + 4 * g + (e & 3);
            float p = fast_exp2(__builtin_fmaf(s[e], c, -lv[e >> 2][e & 3]));
            if (MASK != 0 && !key_visible<MASK>(row0 + r, key, W, G)) p = 0.f;
            s[e] = p;
            dp[e] = p * (dp[e] - dv4[e >> 2][e & 3]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS over two 16-row chunks.
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const int o8 = 8 * kc;
            const s16x8 pf = Op::pack8(s[o8], s[o8 + 1], s[o8 + 2], s[o8 + 3], s[o8 + 4],
                                       s[o8 + 5], s[o8 + 6], s[o8 + 7]);
            const s16x8 sf = Op::pack8(dp[o8], dp[o8 + 1], dp[o8 + 2], dp[o8 + 3], dp[o8 + 4],
                                       dp[o8 + 5], dp[o8 + 6], dp[o8 + 7]);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int base = kc * 16 * C::ROWB;
                const s16x4 glo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(gt + base + tro[0][db]));
                const s16x4 ghi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(gt + base + tro[1][db]));
                dvt[db] = Op::mma(__builtin_shufflevector(glo, ghi, 0, 1, 2, 3, 4, 5, 6, 7), pf,
                                  dvt[db]);
                const s16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(qt + base + tro[0][db]));
                const s16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(qt + base + tro[1][db]));
                dkt[db] = Op::mma(__builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7), sf,
                                  dkt[db]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        if (t + 1 < t1) store_stats(n + 1);
        __syncthreads();
    }

    // dK^T / dV^T: lane (g, key) holds columns db*32 + 8(e/4) + 4g + e%4.
    if (key < Nkv) {
        uint16_t *krow = dK + kvbase + (size_t)key * D;
        uint16_t *vrow = dV + kvbase + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                *(s16x4 *)(krow + db * 32 + 8 * blk + 4 * g) =
                    Op::pack4(dkt[db][4 * blk] * scale, dkt[db][4 * blk + 1] * scale,
                              dkt[db][4 * blk + 2] * scale, dkt[db][4 * blk + 3] * scale);
                *(s16x4 *)(vrow + db * 32 + 8 * blk + 4 * g) =
                    Op::pack4(dvt[db][4 * blk], dvt[db][4 * blk + 1], dvt[db][4 * blk + 2],
                              dvt[db][4 * blk + 3]);
            }
    }
}

template <typename T, int D, int MASK>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ Drow, const float *__restrict__ Lrow, uint16_t *__restrict__ dQ,
    int Nq, int Nkv, float c, float scale, int W, int G, int nqt)
{
    using C = CfgBD<D>;
    using Op = Ops16<T>;
    constexpr int BM = 128, BN = 32, NKK = C::NKK, NDB = C::NDB;
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

    s16x8 qf[NKK], gf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (row < Nq) {
            qf[kk] = *(const s16x8 *)(Q + qbase + (size_t)row * D + 16 * kk + 8 * g);
            gf[kk] = *(const s16x8 *)(dO + qbase + (size_t)row * D + 16 * kk + 8 * g);
        } else {
            qf[kk] = gf[kk] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    const float lrow = row < Nq ? Lrow[(size_t)bh * Nq + row] : INFINITY;
    const float drow = row < Nq ? Drow[(size_t)bh * Nq + row] : 0.f;

    const TileSchedule sch = make_schedule<MASK, BM, BN>(q0, Nq, Nkv, W, G);
    const int ntl = sch.total, nint = sch.interior;
    f32x16 dqt[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqt[db] = f32x16{};

    unsigned off[C::LPW];
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
        const int i = wave + C::NW * u;
        const int r = (i % C::KL) * C::ROWS_PER_LOAD + lane / C::CHUNKS;
        off[u] = r * C::ROWB + 16 * k_swz<D>(r, lane % C::CHUNKS);
    }
    int kofs[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kofs[kk] = li * C::ROWB + 16 * k_swz<D>(li, 2 * kk + g);
    int tro[2][NDB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < NDB; ++db) tro[h][db] = tr_ofs<D>(lane, h, db);

    const char *kb = (const char *)(K + kvbase);
    const char *vb = (const char *)(V + kvbase);
    auto kslot = [&](int n) { return lds + (n & 1) * C::TILEB; };
    auto vslot = [&](int n) { return lds + C::VREG + (n & 1) * C::TILEB; };
    TileSchedule::Cursor cur = sch.begin(), nxt = sch.next(cur);
    if (ntl > 0) {
        issue_kv<C>(kb, vb, off, cur.t * BN, Nkv, kslot(0), vslot(0), wave);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    for (int n = 0; n < ntl; ++n) {
        if (n + 1 < ntl) issue_kv<C>(kb, vb, off, nxt.t * BN, Nkv, kslot(n + 1), vslot(n + 1), wave);
        const char *kt = kslot(n), *vt = vslot(n);
        // S^T = K Q^T and dP^T = V dO^T: lane (g, row) holds keys 8(e/4) + 4g + e%4.
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            s = Op::mma(*(const s16x8 *)(kt + kofs[kk]), qf[kk], s);
            dp = Op::mma(*(const s16x8 *)(vt + kofs[kk]), gf[kk], dp);
        }
        if (n >= nint) mask_tile<MASK>(s, cur.t * BN, ip, Nkv, W, G, g);
#pragma unroll
        for (int e = 0; e < 16; ++e) {  // hidden scores are -inf; P = 0 for any sign of c
            const float p = s[e] == -INFINITY ? 0.f : fast_exp2(__builtin_fmaf(s[e], c, -lrow));
            dp[e] = p * (dp[e] - drow);
        }
        // dQ^T += K^T dS^T over two 16-key chunks.
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
        cur = nxt;
        nxt = sch.next(nxt);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    if (row < Nq) {
        uint16_t *out = dQ + qbase + (size_t)row * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
                *(s16x4 *)(out + db * 32 + 8 * blk + 4 * g) =
                    Op::pack4(dqt[db][4 * blk] * scale, dqt[db][4 * blk + 1] * scale,
                              dqt[db][4 * blk + 2] * scale, dqt[db][4 * blk + 3] * scale);
    }
}

template <typename T, int D, int MASK>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s)
{
    using C = CfgBD<D>;
    const long rows = (long)a.B * a.H * a.Nq;
    float *drow = (float *)a.workspace;
    float *lrow = drow + rows;
    hipLaunchKernelGGL((bwd_rowdot_kernel<T, D>), dim3((unsigned)((rows + 15) / 16)), dim3(256),
                       0, s, (const uint16_t *)a.o, (const uint16_t *)a.dout, a.lse, drow, lrow,
                       rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float c = a.scale * kLog2e;
    const int nkt = (a.Nkv + 127) / 128;
    const int lds_a = C::LDS_BYTES + 512;
    auto ka = bwd_dkdv_kernel<T, D, MASK>;
    e = hipFuncSetAttribute((const void *)ka, hipFuncAttributeMaxDynamicSharedMemorySize, lds_a);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ka, dim3((unsigned)((long)nkt * a.B * a.H)), dim3(256), lds_a, s,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       (const uint16_t *)a.dout, drow, lrow, (uint16_t *)a.dk, (uint16_t *)a.dv,
                       a.Nq, a.Nkv, c, a.scale, a.window, a.n_global, nkt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nqt = (a.Nq + 127) / 128;
    auto kb = bwd_dq_kernel<T, D, MASK>;
    e = hipFuncSetAttribute((const void *)kb, hipFuncAttributeMaxDynamicSharedMemorySize,
                            C::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kb, dim3((unsigned)((long)nqt * a.B * a.H)), dim3(256), C::LDS_BYTES, s,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       (const uint16_t *)a.dout, drow, lrow, (uint16_t *)a.dq, a.Nq, a.Nkv, c,
                       a.scale, a.window, a.n_global, nqt);
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
    default: return launch_bwd<T, D, 4>(a, s);
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
