// Backward pass of bf16 exact attention on gfx950, with recomputation.
//
// Method: the gradients of O = softmax(scale Q K^T) V by the chain rule, with the
// probability matrix recomputed from Q, K and the forward's per-row statistics instead of
// being stored (page "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention": the forward
// keeps only O(N) statistics in HBM, section "FlashAttention-1 (İki Geçişli Yaklaşım)",
// and intermediates are recomputed rather than saved for the backward pass, glossary
// entry "Flash Attention", yapayzekasozluk.tr/etiket/attention). Per (b, h), with
// P = exp(scale S - lse):
//   D_i = sum_d dO[i][d] O[i][d]                     (delta_kernel)
//   dP = dO V^T,  dS = P * (dP - D)                  (row-wise softmax Jacobian)
//   dV = P^T dO,  dK = scale dS^T Q                  (dkdv_kernel)
//   dQ = scale dS K                                  (dq_kernel)
// Under GQA a K/V head's dK and dV sum over the g query heads that read it.
//
// gfx950 mapping (this design):
// * dkdv_kernel: a work-group owns 128 keys of one (batch, KV head) (32 per wave, the
//   wave's K and V rows held in registers) and sweeps every query tile of 32 rows of the
//   g heads of its group, staged in LDS (Q, dO and the rows' lse and D, double-buffered,
//   loaded straight from HBM). Per tile and wave: S = Q K^T on v_mfma_f32_32x32x16_bf16
//   (Q rows from LDS as A, K from registers as B), so each lane owns one key column;
//   P = exp(scale S - lse); dV^T += dO^T P; dP = dO V^T; dS = P (dP - D); dK^T += Q^T dS
//   (transposed tiles through ds_read_b64_tr_b16, P and dS packed to bf16 from the score
//   registers) — in that order, so S/P and dP are never live together and two waves fit
//   per SIMD. Causal: query tiles wholly before the block's first key are skipped.
// * Q, dO and K tiles are read both as rows and transposed; their 16-byte chunks use the
//   kt_swz swizzle, conflict-free for both patterns.
// * dq_kernel: like the forward, a work-group owns 128 query rows (32 per wave, Q and dO
//   rows in registers) and sweeps 64-key tiles of K and V in LDS: S^T = K Q^T,
//   dP^T = V dO^T, dS^T = P^T * (dP^T - D), dQ^T += K^T dS^T (K^T through transposing
//   reads). Each lane owns one query, so lse and D are one value per lane.
// * No atomics: dK/dV and dQ come from separate sweeps (dQ recomputes S and dP), so the
//   result is deterministic. Gradients are accumulated in fp32 and stored as bf16.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "prefill_common.h"

namespace kvfa {
namespace {
using namespace prefill;

// ---- D = rowsum(dO * O) ----------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* __restrict__ o,
                                                    const uint16_t* __restrict__ dout,
                                                    float* __restrict__ delta, long long rows) {
    constexpr int CH = D / 8;  // 16-byte chunks per row
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long row = t / CH;
    const int c = (int)(t % CH);
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + c * 8);
        const u32x4 b = *reinterpret_cast<const u32x4*>(dout + row * D + c * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(bf16lo(a[e]), bf16lo(b[e]), acc);
            acc = fmaf(bf16hi(a[e]), bf16hi(b[e]), acc);
        }
    }
#pragma unroll
    for (int m = 1; m < CH; m <<= 1) acc += shfl_xor(acc, m);
    if (row < rows && c == 0) delta[row] = acc;
}

// 4-byte elements from a buffer straight into LDS: lane L writes lds_base + 4 L.
__device__ __forceinline__ void buf_load4_lds(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                              uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_base, 4, voff, soff, 0, 0);
#endif
}

#ifndef DKDV_WAVES
#define DKDV_WAVES 2
#endif
#ifndef BWD_AHEAD
#define BWD_AHEAD 2
#endif
#ifndef DQ_AHEAD
#define DQ_AHEAD 2
#endif

template <int D>
struct BwdTile {
    static constexpr int ROW = D * 2;        // bytes per row
    static constexpr int KS = D / 16;        // MFMA k-steps over the head dimension
    static constexpr int DB = D / 32;        // 32-dim blocks of a transposed gradient
    static constexpr int BQ = 32;            // query rows per tile (dkdv_kernel)
    static constexpr int QT = BQ * ROW;      // bytes of one Q (or dO) tile
    static constexpr int QDMA = QT / 1024 / 4;  // 1 KiB direct loads per wave per tile
    static constexpr int BK = 64;            // keys per tile (dq_kernel)
    static constexpr int KT = BK * ROW;      // bytes of one K (or V) tile
    static constexpr int KDMA = KT / 1024 / 4;
    static_assert(QDMA >= 1 && KDMA >= 1, "whole 1 KiB loads per wave");
};

// Per-lane LDS offsets of a row-major tile with 16-byte chunks swizzled by kt_swz:
// the A operand of a 32x32x16 MFMA read as rows (row = 32 kb + col, chunk 2s + g), and
// the same tile read transposed (ds_read_b64_tr_b16; rows 16t + 4(G/2) + e and those
// plus 8, chunk 4db + 2(G%2) + a/2, byte 8(a%2), G = lane/16, lane%16 = a + 4e).
// The logical chunk is a constant part (2s, 4db: high bits) OR'ed with a per-lane part
// (low bits), so its XOR with the swizzle is the constant part XOR (per-lane part ^
// swizzle): each offset is two instructions from two per-lane values, instead of one
// register per k-step held across the loop.
template <int D>
struct TileReads {
    int row_base, row_x;            // col * ROW, g ^ kt_swz(col)
    int tr_base0, tr_x0;            // rows 16t + vrow
    int tr_base1, tr_x1;            // rows 16t + vrow + 8
    __device__ __forceinline__ void init(int lane) {
        constexpr int ROW = D * 2;
        const int col = lane & 31, g = lane >> 5;
        row_base = col * ROW;
        row_x = g ^ kt_swz<D>(col);
        const int vG = lane >> 4, va = lane & 3, ve = (lane >> 2) & 3;
        const int vrow = (vG >> 1) * 4 + ve;
        const int lcb = 2 * (vG & 1) + (va >> 1);
        tr_base0 = vrow * ROW + 8 * (va & 1);
        tr_x0 = lcb ^ kt_swz<D>(vrow);
        tr_base1 = (vrow + 8) * ROW + 8 * (va & 1);
        tr_x1 = lcb ^ kt_swz<D>(vrow + 8);
    }
    __device__ __forceinline__ int row_off(int s) const { return row_base + (((2 * s) ^ row_x) << 4); }
    __device__ __forceinline__ int tr_off0(int db) const { return tr_base0 + (((4 * db) ^ tr_x0) << 4); }
    __device__ __forceinline__ int tr_off1(int db) const { return tr_base1 + (((4 * db) ^ tr_x1) << 4); }
};

// Direct-load offsets: piece i of wave w covers tile bytes [1024 (NP w + i), +1024); lane L
// fills byte 16 L of it: row r, physical chunk pc <- logical chunk pc ^ kt_swz(r) of row r.
template <int D, int NP>
__device__ __forceinline__ void dma_offsets(int w, int lane, uint32_t (&off)[NP]) {
    constexpr int ROW = D * 2;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int byte = 1024 * (NP * w + i) + 16 * lane;
        const int r = byte / ROW, pc = (byte % ROW) / 16;
        off[i] = (uint32_t)(r * ROW + ((pc ^ kt_swz<D>(r)) * 16));
    }
}

// Schedules for a block of N MFMAs whose A operands are LDS reads (R reads per MFMA): the
// reads run AHEAD MFMAs ahead of their use, so the LDS latency overlaps the matrix work
// instead of stalling every MFMA.
// ID keeps each block's pattern apart from the others' (and from the other LDS reads).
// A block is N steps of M MFMAs fed by R reads; the reads run AHEAD steps ahead.
template <int N, int R, int AHEAD, int ID, int M = 1>
__device__ __forceinline__ void sched_reads_ahead() {
    static_assert(N > AHEAD, "block longer than the read-ahead");
    __builtin_amdgcn_sched_group_barrier(0x100, R * AHEAD, ID);  // DS reads
#pragma unroll
    for (int i = 0; i < N - AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, M, ID);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, R, ID);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, M * AHEAD, ID);
}

// A 16-key (or 16-query) step of a transposed product: reads the 4 + 4 rows of the
// permuted order that the score accumulator layout gives (see TileReads).
__device__ __forceinline__ u32x4 tr_operand(const char* base, int off0, int off1) {
    const u32x2 a0 = lds_read_tr(base + off0);
    const u32x2 a1 = lds_read_tr(base + off1);
    return u32x4{a0[0], a0[1], a1[0], a1[1]};
}

// ---- dK, dV ------------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DKDV_WAVES, DKDV_WAVES)))
void dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                 const float* __restrict__ lse, const float* __restrict__ delta,
                 uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int H, int Hkv, int Nq,
                 int Nk, int n_kb, float scale, float scale_log2) {
    using T = BwdTile<D>;
    __shared__ __attribute__((aligned(1024))) char qs0[T::QT];
    __shared__ __attribute__((aligned(1024))) char qs1[T::QT];
    __shared__ __attribute__((aligned(1024))) char ds0[T::QT];
    __shared__ __attribute__((aligned(1024))) char ds1[T::QT];
    __shared__ __attribute__((aligned(256))) float st0[2][64];  // lse, D of the tile's rows
    __shared__ __attribute__((aligned(256))) float st1[2][64];
    // d = 128: each wave's 32 K rows stay in LDS (kt_swz-swizzled like the Q tiles) instead
    // of 32 registers per lane, which buys the registers that let the LDS operand reads run
    // ahead of the MFMAs (two work-groups per CU still fit: 65 KiB each).
    constexpr bool KLDS = D == 128;
    __shared__ __attribute__((aligned(1024))) char krow[KLDS ? 4 : 1][KLDS ? T::QT : 1024];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, g = lane >> 5;
    // Key blocks vary slowest: under causal masking block kb sees the most query tiles
    // when kb is small, so the longest work-groups are dispatched first.
    const int n_bk = gridDim.x / n_kb;
    const int kb = blockIdx.x / n_bk;
    const int bk = blockIdx.x % n_bk;  // b * Hkv + kvh
    const int b = bk / Hkv, kvh = bk % Hkv;
    const int gq = H / Hkv;
    const int k0 = kb * 128;
    const int key = k0 + 32 * w + col;  // this lane's key column
    const int off = Nk - Nq;

    // The wave's K and V rows as B operands: K[key][16s + 8g .. +7].
    const auto rk = make_rsrc(k + (size_t)bk * Nk * D, (uint32_t)Nk * D * 2);
    const auto rv = make_rsrc(v + (size_t)bk * Nk * D, (uint32_t)Nk * D * 2);
    u32x4 kf[KLDS ? 1 : T::KS], vf[T::KS];
#pragma unroll
    for (int s = 0; s < T::KS; ++s) {
        if constexpr (!KLDS) kf[s] = buf_load16(rk, (uint32_t)(key * D + 16 * s + 8 * g) * 2);
        vf[s] = buf_load16(rv, (uint32_t)(key * D + 16 * s + 8 * g) * 2);
    }
    char* const kw = krow[KLDS ? w : 0];
    if constexpr (KLDS) {  // rows k0 + 32 w .. +31 into this wave's region (read after a barrier)
        uint32_t koff[T::QT / 1024];
        dma_offsets<D, T::QT / 1024>(0, lane, koff);
#pragma unroll
        for (int i = 0; i < T::QT / 1024; ++i)
            buf_load16_lds(rk, kw + 1024 * i, koff[i], (uint32_t)(k0 + 32 * w) * (uint32_t)T::ROW);
    }

    // Query tiles: causal rows before k0 - off never see this block's keys.
    const int n_qt = (Nq + T::BQ - 1) / T::BQ;
    const int qt0 = CAUSAL ? min(n_qt, max(0, k0 - off) / T::BQ) : 0;
    const int per_head = n_qt - qt0;
    const int n_tiles = gq * per_head;

    uint32_t dq_off[T::QDMA];
    dma_offsets<D, T::QDMA>(w, lane, dq_off);
    TileReads<D> rd;
    rd.init(lane);

    // Tiles go head by head, query tile by query tile: (head offset hq, query tile qt),
    // advanced by a counter instead of a division per tile.
    auto advance = [&](int& hq, int& qt) {
        if (++qt == n_qt) {
            qt = qt0;
            ++hq;
        }
    };
    auto load_tile = [&](int hq, int qt, char* qdst, char* ddst, float (*sdst)[64]) {
        const int h = kvh * gq + hq;
        const size_t pair = (size_t)b * H + h;
        const auto rq = make_rsrc(q + pair * Nq * D, (uint32_t)Nq * D * 2);
        const auto rdo = make_rsrc(dout + pair * Nq * D, (uint32_t)Nq * D * 2);
#pragma unroll
        for (int i = 0; i < T::QDMA; ++i) {
            buf_load16_lds(rq, qdst + 1024 * (T::QDMA * w + i), dq_off[i], (uint32_t)(qt * T::QT));
            buf_load16_lds(rdo, ddst + 1024 * (T::QDMA * w + i), dq_off[i], (uint32_t)(qt * T::QT));
        }
        if (w == 0) {  // the rows' lse and D (lanes past the tile read the next rows)
            const auto rl = make_rsrc(lse + pair * Nq, (uint32_t)Nq * 4);
            const auto rd2 = make_rsrc(delta + pair * Nq, (uint32_t)Nq * 4);
            buf_load4_lds(rl, sdst[0], (uint32_t)lane * 4, (uint32_t)(qt * T::BQ * 4));
            buf_load4_lds(rd2, sdst[1], (uint32_t)lane * 4, (uint32_t)(qt * T::BQ * 4));
        }
    };

    f32x16 dka[T::DB], dva[T::DB];
#pragma unroll
    for (int i = 0; i < T::DB; ++i) {
        dka[i] = f32x16{};
        dva[i] = f32x16{};
    }

    auto tile = [&](int qt, const char* qst, const char* dst, const float (*sst)[64]) {
        const int q0 = qt * T::BQ;
        // S[q][key]: lane holds rows q = 8(i/4) + 4g + i%4 of its key column.
        f32x16 sa = f32x16{};
#pragma unroll
        for (int s = 0; s < T::KS; ++s) {
            const u32x4 aq = *reinterpret_cast<const u32x4*>(qst + rd.row_off(s));
            if constexpr (KLDS) {
                const u32x4 bk = *reinterpret_cast<const u32x4*>(kw + rd.row_off(s));
                sa = mfma32x32x16(aq, bk, sa);
            } else {
                sa = mfma32x32x16(aq, kf[s], sa);
            }
        }
        sched_reads_ahead<T::KS, KLDS ? 2 : 1, BWD_AHEAD, 1>();
        // P = exp(scale s - lse), zero outside the mask and past Nq; packed for the
        // 16-query steps (rows 16t' + 4g + {0..3}, then 16t' + 8 + 4g + {0..3}).
        u32x4 pp[2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // row group r: rows 8r + 4g + 0..3
            const int rl = 8 * r + 4 * g;
            const f32x4 lv = *reinterpret_cast<const f32x4*>(&sst[0][rl]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sa[4 * r + e] = fast_exp2(fmaf(sa[4 * r + e], scale_log2, -lv[e] * kLog2e));
        }
        // Only tiles that reach past Nq or cross the causal diagonal of the block's keys
        // need the mask (a uniform branch; the exponentials above are computed either way,
        // then selected: a conditional exponential becomes a branch per element).
        const bool whole = q0 + T::BQ <= Nq && (!CAUSAL || q0 + off >= k0 + 127);
        if (!whole) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int qa = q0 + 8 * r + 4 * g + e;
                    bool ok = qa < Nq;
                    if (CAUSAL) ok = ok && key <= qa + off;
                    sa[4 * r + e] = ok ? sa[4 * r + e] : 0.f;
                }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tt = r >> 1, half = (r & 1) * 2;
            pp[tt][half] = pack_bf16x2(sa[4 * r], sa[4 * r + 1]);
            pp[tt][half + 1] = pack_bf16x2(sa[4 * r + 2], sa[4 * r + 3]);
        }
        // dV^T += dO^T P (dO^T through transposing reads).
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
                const u32x4 ado = tr_operand(dst + tt * 16 * T::ROW, rd.tr_off0(db), rd.tr_off1(db));
                dva[db] = mfma32x32x16(ado, pp[tt], dva[db]);
            }
        sched_reads_ahead<2 * T::DB, 2, BWD_AHEAD, 2>();
        // dP[q][key] = dO V^T, then dS = P (dP - D), packed like P.
        f32x16 pa = f32x16{};
#pragma unroll
        for (int s = 0; s < T::KS; ++s) {
            const u32x4 ad = *reinterpret_cast<const u32x4*>(dst + rd.row_off(s));
            pa = mfma32x32x16(ad, vf[s], pa);
        }
        sched_reads_ahead<T::KS, 1, BWD_AHEAD, 3>();
        u32x4 ps[2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = 8 * r + 4 * g;
            const f32x4 dv4 = *reinterpret_cast<const f32x4*>(&sst[1][rl]);
            float sv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[e] = sa[4 * r + e] * (pa[4 * r + e] - dv4[e]);
            const int tt = r >> 1, half = (r & 1) * 2;
            ps[tt][half] = pack_bf16x2(sv[0], sv[1]);
            ps[tt][half + 1] = pack_bf16x2(sv[2], sv[3]);
        }
        // dK^T += Q^T dS (Q^T through transposing reads).
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
                const u32x4 aq = tr_operand(qst + tt * 16 * T::ROW, rd.tr_off0(db), rd.tr_off1(db));
                dka[db] = mfma32x32x16(aq, ps[tt], dka[db]);
            }
        sched_reads_ahead<2 * T::DB, 2, BWD_AHEAD, 4>();
    };

    if (n_tiles > 0) {
        int ld_hq = 0, ld_qt = qt0;  // next tile to load
        int cp_hq = 0, cp_qt = qt0;  // next tile to compute
        load_tile(ld_hq, ld_qt, qs0, ds0, st0);
        advance(ld_hq, ld_qt);
        __syncthreads();
        for (int t = 0; t < n_tiles; t += 2) {
            if (t + 1 < n_tiles) {
                load_tile(ld_hq, ld_qt, qs1, ds1, st1);
                advance(ld_hq, ld_qt);
            }
            tile(cp_qt, qs0, ds0, st0);
            advance(cp_hq, cp_qt);
            __syncthreads();
            if (t + 1 < n_tiles) {
                if (t + 2 < n_tiles) {
                    load_tile(ld_hq, ld_qt, qs0, ds0, st0);
                    advance(ld_hq, ld_qt);
                }
                tile(cp_qt, qs1, ds1, st1);
                advance(cp_hq, cp_qt);
                __syncthreads();
            }
        }
    }

    // dK = scale dK^T^T, dV = dV^T^T: lane writes 4 consecutive dims of its key's row.
    if (key < Nk) {
        uint16_t* dkrow = dk + ((size_t)bk * Nk + key) * D;
        uint16_t* dvrow = dv + ((size_t)bk * Nk + key) * D;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d0 = db * 32 + r * 8 + g * 4;
                const u32x2 kp = {pack_bf16x2(dka[db][4 * r] * scale, dka[db][4 * r + 1] * scale),
                                  pack_bf16x2(dka[db][4 * r + 2] * scale, dka[db][4 * r + 3] * scale)};
                const u32x2 vp = {pack_bf16x2(dva[db][4 * r], dva[db][4 * r + 1]),
                                  pack_bf16x2(dva[db][4 * r + 2], dva[db][4 * r + 3])};
                *reinterpret_cast<u32x2*>(dkrow + d0) = kp;
                *reinterpret_cast<u32x2*>(dvrow + d0) = vp;
            }
    }
}

// ---- dQ ----------------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
               const float* __restrict__ lse, const float* __restrict__ delta,
               uint16_t* __restrict__ dq, int H, int Hkv, int Nq, int Nk, int n_qt, int BH,
               float scale, float scale_log2) {
    using T = BwdTile<D>;
    constexpr int BN = T::BK;
    constexpr int KB = BN / 32, PS = BN / 16;
    __shared__ __attribute__((aligned(1024))) char ks0[T::KT];
    __shared__ __attribute__((aligned(1024))) char ks1[T::KT];
    __shared__ __attribute__((aligned(1024))) char vs0[T::KT];
    __shared__ __attribute__((aligned(1024))) char vs1[T::KT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, g = lane >> 5;
    int pair, qt;
    map_work(blockIdx.x, n_qt, BH, H / Hkv, CAUSAL, pair, qt);
    const int b = pair / H, h = pair % H;
    const int kvh = h / (H / Hkv);
    const int q0 = qt * 128;
    const int off = Nk - Nq;
    const int qrow = q0 + w * 32 + col;

    const auto rq = make_rsrc(q + (size_t)pair * Nq * D, (uint32_t)Nq * D * 2);
    const auto rdo = make_rsrc(dout + (size_t)pair * Nq * D, (uint32_t)Nq * D * 2);
    u32x4 qf[T::KS], dof[T::KS];
#pragma unroll
    for (int s = 0; s < T::KS; ++s) {
        qf[s] = buf_load16(rq, (uint32_t)(qrow * D + s * 16 + g * 8) * 2);
        dof[s] = buf_load16(rdo, (uint32_t)(qrow * D + s * 16 + g * 8) * 2);
    }
    const bool valid_row = qrow < Nq;
    const float lse2 = valid_row ? lse[(size_t)pair * Nq + qrow] * kLog2e : 0.f;
    const float drow = valid_row ? delta[(size_t)pair * Nq + qrow] : 0.f;

    const int n_all = (Nk + BN - 1) / BN;
    int n_tiles = n_all;
    if (CAUSAL) {
        const int last_row = min(q0 + 128, Nq) - 1;
        n_tiles = min(n_all, (last_row + off) / BN + 1);
    }

    const auto rk = make_rsrc(k + ((size_t)b * Hkv + kvh) * Nk * D, (uint32_t)Nk * D * 2);
    const auto rv = make_rsrc(v + ((size_t)b * Hkv + kvh) * Nk * D, (uint32_t)Nk * D * 2);
    uint32_t dk_off[T::KDMA];
    dma_offsets<D, T::KDMA>(w, lane, dk_off);
    auto load_kv = [&](int j, char* kd, char* vd) {
#pragma unroll
        for (int i = 0; i < T::KDMA; ++i) {
            buf_load16_lds(rk, kd + 1024 * (T::KDMA * w + i), dk_off[i], (uint32_t)(j * T::KT));
            buf_load16_lds(rv, vd + 1024 * (T::KDMA * w + i), dk_off[i], (uint32_t)(j * T::KT));
        }
    };
    TileReads<D> rd;
    rd.init(lane);

    f32x16 dqa[T::DB];
#pragma unroll
    for (int i = 0; i < T::DB; ++i) dqa[i] = f32x16{};

    // Tiles below the work-group's first row's diagonal (and below Nk) need no mask when
    // all its rows exist.
    int n_plain = q0 + 127 < Nq ? Nk / BN : 0;
    if (CAUSAL) n_plain = min(n_plain, (q0 + off + 1) / BN);

    auto tile = [&](int j, const char* kst, const char* vst, auto masked)
                    __attribute__((always_inline)) {
        f32x16 sa[KB], pa[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            sa[kb] = f32x16{};
            pa[kb] = f32x16{};
#pragma unroll
            for (int s = 0; s < T::KS; ++s) {
                const u32x4 ak = *reinterpret_cast<const u32x4*>(kst + rd.row_off(s) + kb * 32 * T::ROW);
                const u32x4 av = *reinterpret_cast<const u32x4*>(vst + rd.row_off(s) + kb * 32 * T::ROW);
                sa[kb] = mfma32x32x16(ak, qf[s], sa[kb]);
                pa[kb] = mfma32x32x16(av, dof[s], pa[kb]);
            }
        }
        sched_reads_ahead<KB * T::KS, 2, DQ_AHEAD, 5, 2>();
        // dS^T for key rows 32kb + 8(i/4) + 4g + i%4 of this lane's query, packed for the
        // 16-key steps (rows 16t + 4g + {0..3}, then 16t + 8 + 4g + {0..3}).
        const int lim = CAUSAL ? min(Nk - 1, qrow + off) - j * BN - 4 * g : Nk - 1 - j * BN - 4 * g;
#pragma unroll
        for (int t = 0; t < PS; ++t) {
            const int kb = t >> 1, base = (t & 1) * 8;
            u32x4 ps;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float sv[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int i = base + 2 * u + e;
                    const int kk = kb * 32 + (i >> 2) * 8 + (i & 3);
                    const float ex = fast_exp2(fmaf(sa[kb][i], scale_log2, -lse2));
                    float p = ex;
                    if constexpr (decltype(masked)::value)
                        p = (valid_row && kk <= lim) ? ex : 0.f;  // selected, not branched
                    sv[e] = p * (pa[kb][i] - drow);
                }
                ps[u] = pack_bf16x2(sv[0], sv[1]);
            }
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
                const u32x4 a = tr_operand(kst + t * 16 * T::ROW, rd.tr_off0(db), rd.tr_off1(db));
                dqa[db] = mfma32x32x16(a, ps, dqa[db]);
            }
        }
    };

    // Tile j (stage j & 1) with the next tile's K and V loaded meanwhile.
    auto step = [&](int j, auto par, auto masked) __attribute__((always_inline)) {
        constexpr int pv = decltype(par)::value;
        if (j + 1 < n_tiles) load_kv(j + 1, pv ? ks0 : ks1, pv ? vs0 : vs1);
        tile(j, pv ? ks1 : ks0, pv ? vs1 : vs0, masked);
        __syncthreads();
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    load_kv(0, ks0, vs0);
    __syncthreads();
    // Unmasked tiles two at a time (stage parity alternates), then the rest with masking.
    int j = 0;
    for (; j + 1 < n_plain; j += 2) {
        step(j, P0{}, std::false_type{});
        step(j + 1, P1{}, std::false_type{});
    }
    for (; j < n_tiles; j += 2) {
        step(j, P0{}, std::true_type{});
        if (j + 1 < n_tiles) step(j + 1, P1{}, std::true_type{});
    }

    if (valid_row) {
        uint16_t* drow_out = dq + ((size_t)pair * Nq + qrow) * D;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d0 = db * 32 + r * 8 + g * 4;
                const u32x2 pk = {pack_bf16x2(dqa[db][4 * r] * scale, dqa[db][4 * r + 1] * scale),
                                  pack_bf16x2(dqa[db][4 * r + 2] * scale, dqa[db][4 * r + 3] * scale)};
                *reinterpret_cast<u32x2*>(drow_out + d0) = pk;
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_typed(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            int B, int H, int Hkv, int Nq, int Nk, float scale, float* delta,
                            hipStream_t stream) {
    const float scale_log2 = scale * kLog2e;
    const long long rows = (long long)B * H * Nq;
    const long long threads = rows * (D / 8);
    hipLaunchKernelGGL(delta_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const uint16_t*>(o),
                       static_cast<const uint16_t*>(dout), delta, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_kb = (Nk + 127) / 128;
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3(n_kb * B * Hkv), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), lse,
                       delta, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), H, Hkv, Nq,
                       Nk, n_kb, scale, scale_log2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_qt = (Nq + 127) / 128;
    hipLaunchKernelGGL((dq_kernel<D, CAUSAL>), dim3(n_qt * B * H), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), lse,
                       delta, static_cast<uint16_t*>(dq), H, Hkv, Nq, Nk, n_qt, B * H, scale,
                       scale_log2);
    return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int Nq) { return (size_t)B * H * Nq * sizeof(float); }

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           void* workspace, hipStream_t stream) {
    float* delta = static_cast<float*>(workspace);
    if (d == 128)
        return causal ? launch_bwd_typed<128, true>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv,
                                                    Nq, Nk, scale, delta, stream)
                      : launch_bwd_typed<128, false>(q, k, v, o, lse, dout, dq, dk, dv, B, H,
                                                     Hkv, Nq, Nk, scale, delta, stream);
    return causal ? launch_bwd_typed<64, true>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, Nq,
                                               Nk, scale, delta, stream)
                  : launch_bwd_typed<64, false>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, Nq,
                                                Nk, scale, delta, stream);
}

}  // namespace kvfa
