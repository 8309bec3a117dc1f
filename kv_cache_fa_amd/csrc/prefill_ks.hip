// bf16 exact attention (prefill) for launches too small to fill the chip with 256-row
// work-groups: each work-group owns 64 query rows of one (batch, head), and its key range
// is split into four parts that run side by side.
//
// Method (page "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention"): the same tiling and
// online softmax as the other prefill kernels ("FlashAttention'ın Temelleri", "Online
// Softmax Prensibi" steps 1-5). The keys of a row are cut into parts, each part keeps its
// own running max m, sum l and unnormalised output, and the parts are merged at the end
// with the rule the page gives for merging two blocks' statistics: m = max(m_a, m_b),
// l = e^(m_a - m) l_a + e^(m_b - m) l_b, and the same factors on the outputs.
//
// Block sizes by launch size (section "FlashAttention-2: Optimizasyonlar ve
// İyileştirmeler", item 4: the block size is picked per hardware and sequence length;
// item 1: one head's work is spread over more compute units). The 256-row work-groups of
// the ping-pong kernel each sweep their row block's whole key range, so when there are
// few of them the launch lasts as long as the longest sweep while most compute units idle
// (B2 H8 N1024 d64 causal: 64 work-groups, each up to 16 tiles of 64 keys one after the
// other). Here the longest chain is a quarter of that, with 4x as many work-groups.
//
// gfx950 mapping:
// * 512 threads = 8 waves: row group rg (32 rows) x key part p; part p takes key tiles
//   p, p + 4, p + 8, ... (64 keys for d = 64, 32 for d = 128). The two waves of a part
//   (one per row group) share its K and V tiles: each loads half of them straight into
//   LDS (buffer_load ... lds), double-buffered; a work-group barrier per step publishes
//   the next tiles. Sharing halves the K/V reads of a four-wave, 32-row design (whose
//   waves each loaded their own tiles): B2 H8 N1024 d64 causal 14.8 -> 10.2 us.
// * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K rows from LDS as A (16-byte chunks
//   XOR-swizzled by row), the wave's 32 Q rows held as B (each row group's Q tile is
//   loaded once into LDS for its four parts and read from there: 10.3 -> 9.8 us on B2 H8
//   N1024 d64 causal); each lane owns one query column, so the row max is in-lane plus
//   one exchange with lane ^ 32.
// * O^T += V^T P^T: V^T through transposing LDS reads (ds_read_b64_tr_b16), swizzled so
//   they are conflict-free; P^T straight from the score registers.
// * Loads of tiles past the work-group's last one go through zero-size descriptors
//   (nothing is fetched), so every step issues the same loads.
// * Merge: every wave writes its (m, l) per row and its fp32 accumulator to LDS over the
//   K/V stages; after a barrier wave (rg, p) combines dims 32 db + 8 p + {0..7} of its
//   row group's four parts and stores them as bf16, and part 0 stores lse = m + ln l.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "prefill_common.h"

namespace kvfa {

namespace {
using namespace prefill;

template <int D>
struct TileKS {
    static constexpr int RG = 2;                 // row groups (32 rows each)
    static constexpr int KP = 4;                 // key parts
    static constexpr int NW = RG * KP;           // waves per work-group
    static constexpr int NT = 64 * NW;           // threads per work-group
    static constexpr int BM = 32 * RG;           // query rows per work-group
    static constexpr int BN = D == 64 ? 64 : 32; // keys per tile
    static constexpr int KB = BN / 32;           // 32-key blocks of S^T
    static constexpr int KS = D / 16;            // MFMA k-steps of Q.K (16 dims each)
    static constexpr int DB = D / 32;            // 32-dim blocks of O^T
    static constexpr int PS = BN / 16;           // MFMA k-steps of P.V (16 keys each)
    static constexpr int ROW = D * 2;            // bytes per K/V row
    static constexpr int TILE = BN * ROW;        // bytes of one K (or V) tile
    static constexpr int HALF = TILE / 1024 / RG;  // 1 KiB direct loads per wave per tile
    static constexpr int PART = DB * 16 * 64 * 4;  // bytes of one wave's fp32 accumulator
    static_assert(HALF >= 1 && HALF * 1024 * RG == TILE, "whole 1 KiB loads per wave");
    static_assert(PART <= 2 * TILE, "merge area fits in a part's stages");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_ks_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                   float* __restrict__ lse, int H, int Hkv, int Nq, int Nk, int n_qt, int BH,
                   float scale_log2, float tau_raw) {
    using T = TileKS<D>;
    constexpr int BN = T::BN;
    // Stage s of key part p: K in ks<s>[p], V in vs<s>[p] (separate arrays, so the compiler
    // can tell a load into one stage from reads of the other); reused for the merge.
    // 128 KiB (+ the Q tiles): one work-group per CU, two waves per SIMD.
    __shared__ __attribute__((aligned(1024))) char ks0[T::KP][T::TILE];
    __shared__ __attribute__((aligned(1024))) char ks1[T::KP][T::TILE];
    __shared__ __attribute__((aligned(1024))) char vs0[T::KP][T::TILE];
    __shared__ __attribute__((aligned(1024))) char vs1[T::KP][T::TILE];
    __shared__ float red[T::NW][2][32];  // per wave: m (log2 units) and l of each row
    // Each row group's 32 Q rows, loaded once for its four parts (16-byte chunks swizzled
    // by row like the K tiles, so the 32 rows read together hit different banks).
    __shared__ __attribute__((aligned(1024))) char qs[T::RG][32 * T::ROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kp = w & (T::KP - 1);   // key part
    const int rg = w / T::KP;         // row group
    const int col = lane & 31;        // query row (column of S^T) owned by this lane
    const int g = lane >> 5;          // which half of the MFMA k-slots this lane supplies

    int pair, qt;
    map_work(blockIdx.x, n_qt, BH, H / Hkv, CAUSAL, pair, qt);
    const int b = pair / H, h = pair % H;
    const int kvh = h / (H / Hkv);
    const int q0 = qt * T::BM;
    const int off = Nk - Nq;
    const int qrow = q0 + 32 * rg + col;

    const auto rq = make_rsrc(q + (size_t)pair * Nq * D, (uint32_t)Nq * D * 2);
    const auto rk = make_rsrc(k + ((size_t)b * Hkv + kvh) * Nk * D, (uint32_t)Nk * D * 2);
    const auto rv = make_rsrc(v + ((size_t)b * Hkv + kvh) * Nk * D, (uint32_t)Nk * D * 2);
    // Zero-size descriptors for the loads of tiles past the last one: nothing is fetched.
    const auto rk_none = make_rsrc(k, 0u);
    const auto rv_none = make_rsrc(v, 0u);

    // Key tiles of the work-group's rows, and this wave's first tile that needs a mask.
    const int n_all = (Nk + BN - 1) / BN;
    int n_tiles = n_all, full = Nk / BN;
    if (CAUSAL) {
        const int last_row = min(q0 + T::BM, Nq) - 1;
        n_tiles = min(n_all, (last_row + off) / BN + 1);
        full = min(full, (q0 + 32 * rg + off + 1) / BN);
    }
    const int steps = (n_tiles + T::KP - 1) / T::KP;  // part p takes tiles p, p + 4, ...

    // B operand of S^T = K Q^T: Q[qrow][16 s + 8 g .. +7]; rows past Nq load as zero.
    // The row group's tile arrives by direct loads (part p fills 1 KiB pieces p, p + 4, ...)
    // before the first barrier, and each wave reads its operands from it after that.
    constexpr int QP = 32 * T::ROW / 1024;  // 1 KiB pieces of a row group's Q tile
    static_assert(QP % T::KP == 0, "whole pieces per part");
#pragma unroll
    for (int i = kp; i < QP; i += T::KP) {
        const int byte = 1024 * i + 16 * lane;
        const int r = byte / T::ROW, pc = (byte % T::ROW) / 16;
        buf_load16_lds(rq, qs[rg] + 1024 * i, (uint32_t)(r * T::ROW + ((pc ^ k_swz<D>(r)) * 16)),
                       (uint32_t)(q0 + 32 * rg) * (uint32_t)T::ROW);
    }
    u32x4 qf[T::KS];

    // Direct loads: this wave fills pieces [HALF rg, HALF rg + HALF) of its part's K and V
    // tiles; lane L of piece i writes tile byte 1024 i + 16 L: row r, physical chunk pc,
    // with logical chunk pc ^ swizzle(r) of row r.
    uint32_t dk_off[T::HALF], dv_off[T::HALF];
#pragma unroll
    for (int i = 0; i < T::HALF; ++i) {
        const int byte = 1024 * (T::HALF * rg + i) + 16 * lane;
        const int r = byte / T::ROW, pc = (byte % T::ROW) / 16;
        dk_off[i] = (uint32_t)(r * T::ROW + ((pc ^ k_swz<D>(r)) * 16));
        dv_off[i] = (uint32_t)(r * T::ROW + ((pc ^ v_swz<D>(r)) * 16));
    }
    auto load = [&](int j, char* kdst, char* vdst) {
        const bool have = j < n_tiles;
        const auto r1 = have ? rk : rk_none;
        const auto r2 = have ? rv : rv_none;
        const uint32_t toff = (uint32_t)j * (uint32_t)T::TILE;
#pragma unroll
        for (int i = 0; i < T::HALF; ++i) {
            buf_load16_lds(r1, kdst + 1024 * (T::HALF * rg + i), dk_off[i], toff);
            buf_load16_lds(r2, vdst + 1024 * (T::HALF * rg + i), dv_off[i], toff);
        }
    };
    // K operand (kb, s): row 32 kb + col, logical chunk 2 s + g.
    int kr_off[T::KS];
#pragma unroll
    for (int s = 0; s < T::KS; ++s) kr_off[s] = col * T::ROW + (((2 * s + g) ^ k_swz<D>(col)) * 16);
    // V^T operand (t, db, half): rows 16 t + 8 half + 4 (G/2) + e, logical chunk
    // 4 db + 2 (G%2) + a/2, byte 8 (a%2) in it (G = lane/16, lane%16 = a + 4 e).
    const int vG = lane >> 4, va = lane & 3, ve = (lane >> 2) & 3;
    const int vrow = (vG >> 1) * 4 + ve;
    int vr_off[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
        vr_off[db] = vrow * T::ROW + (((4 * db + 2 * (vG & 1) + (va >> 1)) ^ v_swz<D>(vrow)) * 16) +
                     8 * (va & 1);

    float m_used = -INFINITY;  // raw-score reference max of this lane's row
    float l_part = 0.f;        // this lane's share of the row sum
    f32x16 oacc[T::DB];
#pragma unroll
    for (int i = 0; i < T::DB; ++i) oacc[i] = f32x16{};

    // One tile: scores, mask (tiles from `full` on), running max, exponentials, P.V.
    auto tile = [&](const int j, const char* kst, const char* vst) {
        f32x16 sacc[T::KB];
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
            sacc[kb] = f32x16{};
#pragma unroll
            for (int s = 0; s < T::KS; ++s) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(kst + kr_off[s] + kb * 32 * T::ROW);
                sacc[kb] = mfma32x32x16(a, qf[s], sacc[kb]);
            }
        }
        if (j >= full) {
            // key offset inside the tile of element (kb, i) is kb*32 + 8*(i/4) + 4g + i%4;
            // it is dead past the row's last key and past Nk.
            int lim = Nk - 1 - j * BN - 4 * g;
            if (CAUSAL) lim = min(lim, qrow + off - j * BN - 4 * g);
#pragma unroll
            for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) sacc[kb][i] = -INFINITY;
        }
        float mx = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        mx = fmaxf(mx, xor32(mx));
        const float m_cand = fmaxf(m_used, mx);
        const bool move = m_cand > m_used + tau_raw;
        if (__builtin_amdgcn_ballot_w64(move)) {
            // Only rows whose max moved change their reference; a row that does not move
            // keeps alpha = 1 (its reference may still be -inf).
            const float m_new = move ? m_cand : m_used;
            const float alpha = move ? fast_exp2((m_used - m_new) * scale_log2) : 1.f;
            m_used = m_new;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        }
        // A row that has seen none of its keys yet (a part that starts past the row's
        // causal limit) keeps a -inf reference; its exponentials are taken against 0,
        // which makes them exp2(-inf) = 0.
        const float mb = m_used == -INFINITY ? 0.f : m_used * scale_log2;
#pragma unroll
        for (int t = 0; t < T::PS; ++t) {
            const int kb = t >> 1, base = (t & 1) * 8;
            u32x4 pf;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float p0 = fast_exp2(fmaf(sacc[kb][base + 2 * u], scale_log2, -mb));
                const float p1 = fast_exp2(fmaf(sacc[kb][base + 2 * u + 1], scale_log2, -mb));
                pf[u] = pack_bf16x2(p0, p1);
                l_part += p0 + p1;  // fp32 sum of the unrounded exponentials
            }
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
                const u32x2 a0 = lds_read_tr(vst + vr_off[db] + (t * 16) * T::ROW);
                const u32x2 a1 = lds_read_tr(vst + vr_off[db] + (t * 16 + 8) * T::ROW);
                const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
                oacc[db] = mfma32x32x16(a, pf, oacc[db]);
            }
        }
    };

    // Step i: part p's tile p + 4 i from stage i & 1, while step i + 1's tiles load into the
    // other stage; the barrier that ends a step completes those loads (both row groups'
    // halves) and frees the stage just read.
    load(kp, ks0[kp], vs0[kp]);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < T::KS; ++s)
        qf[s] = *reinterpret_cast<const u32x4*>(qs[rg] + col * T::ROW +
                                               (((2 * s + g) ^ k_swz<D>(col)) * 16));
    for (int i = 0; i < steps; i += 2) {
        const int j = kp + T::KP * i;
        load(j + T::KP, ks1[kp], vs1[kp]);
        if (j < n_tiles) tile(j, ks0[kp], vs0[kp]);
        __syncthreads();
        if (i + 1 < steps) {
            const int j1 = j + T::KP;
            load(j1 + T::KP, ks0[kp], vs0[kp]);
            if (j1 < n_tiles) tile(j1, ks1[kp], vs1[kp]);
            __syncthreads();
        }
    }

    // ---- merge the four parts of each row group ----
    // All loads are done (the last barrier waited for them). Wave (rg, p)'s accumulator,
    // 1 KiB chunk c = 4 db + r: chunk c of [ks0|ks1][p] (row group 0|1), then of [vs0|vs1][p].
    constexpr int CPT = T::TILE / 1024;
    auto chunk = [&](int rgx, int px, int c) -> char* {
        char* a = c < CPT ? (rgx == 0 ? ks0[px] : ks1[px]) : (rgx == 0 ? vs0[px] : vs1[px]);
        return a + 1024 * (c % CPT);
    };
    const float l = l_part + xor32(l_part);
    if (g == 0) {
        red[w][0][col] = m_used == -INFINITY ? -INFINITY : m_used * scale_log2;
        red[w][1][col] = l;
    }
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<f32x4*>(chunk(rg, kp, 4 * db + r) + 16 * lane) =
                f32x4{oacc[db][4 * r], oacc[db][4 * r + 1], oacc[db][4 * r + 2], oacc[db][4 * r + 3]};
    __syncthreads();

    // Every row attends key 0, which is in part 0's first tile, so M is finite.
    float mw[T::KP], M = -INFINITY;
#pragma unroll
    for (int x = 0; x < T::KP; ++x) {
        mw[x] = red[rg * T::KP + x][0][col];
        M = fmaxf(M, mw[x]);
    }
    float a[T::KP], L = 0.f;
#pragma unroll
    for (int x = 0; x < T::KP; ++x) {
        a[x] = fast_exp2(mw[x] - M);  // 0 for a part that saw no key of the row
        L += a[x] * red[rg * T::KP + x][1][col];
    }
    const float inv = 1.f / L;
    if (qrow < Nq) {
        uint16_t* orow = o + ((size_t)pair * Nq + qrow) * D;
        const int r = kp;  // this wave stores dims 32 db + 8 kp + 4 g .. +3 of its rows
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < T::KP; ++x) {
                const f32x4 p = *reinterpret_cast<const f32x4*>(chunk(rg, x, 4 * db + r) + 16 * lane);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = fmaf(a[x], p[c], acc[c]);
            }
            const u32x2 pk = {pack_bf16x2(acc[0] * inv, acc[1] * inv),
                              pack_bf16x2(acc[2] * inv, acc[3] * inv)};
            *reinterpret_cast<u32x2*>(orow + db * 32 + r * 8 + g * 4) = pk;
        }
        if (lse != nullptr && kp == 0 && g == 0)
            lse[(size_t)pair * Nq + qrow] = (M + fast_log2(L)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_ks(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Hkv, int Nq, int Nk, float scale, hipStream_t stream) {
    using T = TileKS<D>;
    const int n_qt = (Nq + T::BM - 1) / T::BM;
    const int BH = B * H;
    const float scale_log2 = scale * kLog2e;
    const float tau_raw = 8.0f / scale_log2;  // move the reference max past +8 in log2 units
    hipLaunchKernelGGL((fwd_ks_kernel<D, CAUSAL>), dim3(n_qt * BH), dim3(T::NT), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, H, Hkv,
                       Nq, Nk, n_qt, BH, scale_log2, tau_raw);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16_key_split(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int B, int H, int Hkv, int Nq, int Nk, int d,
                                     int causal, float scale, hipStream_t stream) {
    if (d == 128)
        return causal ? launch_ks<128, true>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream)
                      : launch_ks<128, false>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream);
    return causal ? launch_ks<64, true>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream)
                  : launch_ks<64, false>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream);
}

}  // namespace kvfa
