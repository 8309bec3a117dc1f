// bf16 exact attention (prefill) on gfx950 MFMA, fp32 accumulation: the four-wave kernel
// behind the two-pass form (fa_fwd_two_pass). Single-pass prefill (fa_fwd, fa_fwd_window,
// fa_fwd_paged) runs the ping-pong kernel of prefill_pp.hip.
//
// Method (page "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention"):
// * K and V are split into tiles that are staged in LDS, the CU's fast on-chip
//   memory, while the work-group's Q rows stay in registers ("FlashAttention'ın
//   Temelleri": tiling so the N x N score matrix never reaches HBM).
// * Each query row keeps a running max and sum that are merged tile by tile
//   ("Online Softmax Prensibi", steps 1-5); the output accumulator is rescaled by
//   the same factor so one pass over K/V suffices, and it is divided by the row sum
//   once at the end.
// * Work is split over query rows: every work-group owns one Q tile of one (batch,
//   head) and sweeps all of the K/V tiles it needs ("FlashAttention-2:
//   Optimizasyonlar ve İyileştirmeler", item 1); the next K/V tile is fetched from
//   HBM while the current one is being used (item 2).
// * GQA: query head h reads K/V head h / (H / Hkv) (glossary entry "KV Cache
//   (Anahtar-Değer Önbelleği)", yapayzekasozluk.tr/etiket/attention).
//
// gfx950 mapping (this design, not the pages'):
// * 256 threads = 4 waves; each wave owns 32 query rows (BM = 128 rows per
//   work-group); 64 keys per tile. K and V tiles go from HBM straight into LDS
//   (buffer_load ... lds) with XOR-swizzled 16-byte chunks, double-buffered (64 KiB of
//   LDS, two work-groups per CU).
// * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   A = K rows read from LDS, B = the wave's Q held in registers. Each lane then
//   owns one query column, so the row max and row sum are in-lane reductions plus
//   a single exchange with lane ^ 32.
// * The output is also accumulated transposed, O^T += V^T P^T: B = P^T comes
//   straight from the score registers (converted to bf16), A = V^T read from the V
//   tile through transposing LDS reads. The key order inside each 16-key MFMA step
//   follows the score accumulator layout; any order is valid for a sum over keys as
//   long as A and B agree.
// * Softmax uses exp2 with scale*log2(e) folded into one FMA per score. The
//   reference max used for the exponentials is only moved when the true max grows by
//   more than 8 (log2 units); exponentials then stay below 2^8 and the result is
//   unchanged, since softmax(x) = softmax(x - c) for any c ("FlashAttention'ın
//   Temelleri"). The statistics pass computes a tile's max only when the tile's
//   exponentials against the current reference say it may have moved (a lane's share of
//   them summing to more than 128), as the single-pass kernel does, so the two agree bit
//   for bit.
// * Causal: key tiles entirely in a row block's future are never visited; only the
//   tiles crossing the diagonal (and a ragged last tile) pay for masking. Work is
//   ordered longest-first, and each XCD's work-groups share the same (batch, head)
//   group so K/V tiles are reused from that XCD's L2.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "prefill_common.h"

namespace kvfa {

namespace {
using namespace prefill;

template <int D>
struct Tile {
    static constexpr int NT = 256;              // threads per work-group
    static constexpr int BM = 128;              // query rows per work-group (32 per wave)
    static constexpr int BN = 64;               // keys per tile
    static constexpr int CH = D / 8;            // 16-byte chunks per K/V row
    static constexpr int KB = BN / 32;          // 32-key blocks of S^T
    static constexpr int KS = D / 16;           // MFMA k-steps of Q.K (16 dims each)
    static constexpr int DB = D / 32;           // 32-dim blocks of O^T
    static constexpr int PS = BN / 16;          // MFMA k-steps of P.V (16 keys each)
    static constexpr int ROW = D * 2;           // bytes per K/V row (rows are unpadded)
    static constexpr int TILE = BN * ROW;       // bytes of one K (or V) tile
    static constexpr int DMA = TILE / 1024 / (NT / 64);  // 1 KiB direct loads per wave per tile
    static_assert(DMA >= 1 && DMA * 1024 * (NT / 64) == TILE, "whole 1 KiB loads per wave");
};


// Per-iteration schedule of one wave (tile j):
//   issue S_{j+1} = K_{j+1} Q^T on MFMA  |  softmax of S_j on the VALU (mask, running max,
//   rescale, P_j = exp2(...)), then O^T += V_j^T P_j^T on MFMA
// so the MFMAs of the next tile's scores overlap this tile's softmax inside each wave.
// Tiles go from HBM straight into LDS (buffer_load ... lds): K two tiles ahead and V one
// tile ahead, each into one of two stages that are separate LDS arrays, so the compiler
// can tell that the loads in flight never alias the stage being read; the work-group
// barrier that ends tile j (after the loads complete) publishes K_{j+2} and V_{j+1}.
//
// Two passes (PASS = 1, then PASS = 2; page "Donanıma Duyarlı Algoritma Tasarımı:
// FlashAttention", section "FlashAttention-1 (İki Geçişli Yaklaşım)"): the first pass
// sweeps K only and keeps each row's running max and sum, leaving the row statistics in
// HBM as lse = M + ln L; the second recomputes the scores, normalises them directly with
// those statistics (P = exp(scale s - lse)) and accumulates P V, with no rescaling.
template <int D, bool CAUSAL, int PASS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                     float* __restrict__ lse, int H, int Hkv, int Nq, int Nk, int n_qt,
                     int BH, float scale_log2, float tau_raw) {
    static_assert(PASS == 1 || PASS == 2, "statistics pass, then output pass");
    using T = Tile<D>;
    constexpr int BN = T::BN;
    __shared__ __attribute__((aligned(1024))) char ks0[T::TILE];
    __shared__ __attribute__((aligned(1024))) char ks1[T::TILE];
    __shared__ __attribute__((aligned(1024))) char vs0[T::TILE];
    __shared__ __attribute__((aligned(1024))) char vs1[T::TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
    const int col = lane & 31;      // query column of S^T / O^T owned by this lane
    const int g = lane >> 5;        // which half of the k-slots this lane supplies

    int pair, qt;
    map_work(blockIdx.x, n_qt, BH, H / Hkv, CAUSAL, pair, qt);
    const int b = pair / H, h = pair % H;
    const int kvh = h / (H / Hkv);
    const int q0 = qt * T::BM;
    const int off = Nk - Nq;
    const int qrow = q0 + w * 32 + col;

    const auto rq = make_rsrc(q + (size_t)pair * Nq * D, (uint32_t)Nq * D * 2);
    const auto rk = make_rsrc(k + ((size_t)b * Hkv + kvh) * Nk * D, (uint32_t)Nk * D * 2);
    const auto rv = make_rsrc(v + ((size_t)b * Hkv + kvh) * Nk * D, (uint32_t)Nk * D * 2);

    // B operand of S^T = K Q^T: Q[qrow][16s + 8g .. +7]; rows past Nq load as zero.
    u32x4 qf[T::KS];
#pragma unroll
    for (int s = 0; s < T::KS; ++s)
        qf[s] = buf_load16(rq, (uint32_t)(qrow * D + s * 16 + g * 8) * 2);

    // Tiles to visit and the first one that needs a mask.
    const int n_all = (Nk + BN - 1) / BN;
    int n_tiles = n_all, full = Nk / BN;
    if (CAUSAL) {
        const int last_row = min(q0 + T::BM, Nq) - 1;
        n_tiles = min(n_all, (last_row + off) / BN + 1);
        full = min(full, (q0 + off + 1) / BN);
    }

    // Direct loads: the wave's i-th 1 KiB piece of a tile covers tile bytes
    // [1024 (DMA w + i), +1024); lane L fills byte 16 L of it, i.e. row r, physical chunk
    // pc, with logical chunk pc ^ swizzle(r) of row r.
    uint32_t dk_off[T::DMA], dv_off[T::DMA];
#pragma unroll
    for (int i = 0; i < T::DMA; ++i) {
        const int byte = 1024 * (T::DMA * w + i) + 16 * lane;
        const int r = byte / T::ROW, pc = (byte % T::ROW) / 16;
        dk_off[i] = (uint32_t)(r * T::ROW + ((pc ^ k_swz<D>(r)) * 16));
        dv_off[i] = (uint32_t)(r * T::ROW + ((pc ^ v_swz<D>(r)) * 16));
    }
    auto load_k = [&](int j, char* dst) {
#pragma unroll
        for (int i = 0; i < T::DMA; ++i)
            buf_load16_lds(rk, dst + 1024 * (T::DMA * w + i), dk_off[i], (uint32_t)(j * T::TILE));
    };
    auto load_v = [&](int j, char* dst) {
#pragma unroll
        for (int i = 0; i < T::DMA; ++i)
            buf_load16_lds(rv, dst + 1024 * (T::DMA * w + i), dv_off[i], (uint32_t)(j * T::TILE));
    };

    // Per-lane LDS read offsets. K operand (kb, s): row 32 kb + col, logical chunk 2s + g.
    // V^T operand (t, db, half): rows 16t + 8 half + 4(G/2) + e, logical chunk
    // 4 db + 2(G%2) + a/2, byte 8(a%2) in it (G = lane/16, lane%16 = a + 4e).
    int kr_off[T::KS];
#pragma unroll
    for (int s = 0; s < T::KS; ++s)
        kr_off[s] = col * T::ROW + (((2 * s + g) ^ k_swz<D>(col)) * 16);
    const int vG = lane >> 4, va = lane & 3, ve = (lane >> 2) & 3;
    const int vrow = (vG >> 1) * 4 + ve;  // row within a 16-key step (swizzle depends on it only)
    int vr_off[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
        vr_off[db] = vrow * T::ROW + (((4 * db + 2 * (vG & 1) + (va >> 1)) ^ v_swz<D>(vrow)) * 16) +
                     8 * (va & 1);

    // Second pass: the row's statistics in log2 units (rows past Nq are never stored).
    float mb_fixed = 0.f;
    if constexpr (PASS == 2) mb_fixed = qrow < Nq ? lse[(size_t)pair * Nq + qrow] * kLog2e : 0.f;
    float m_used = -INFINITY;  // raw-score reference max of this lane's query
    float l_part = 0.f;        // this lane's share of the row sum
    f32x16 oacc[T::DB];
#pragma unroll
    for (int i = 0; i < T::DB; ++i) oacc[i] = f32x16{};
    // Score accumulators of two consecutive tiles; which one is current alternates with
    // the tile's parity, a compile-time constant at every call site.
    f32x16 sbuf[2][T::KB];

    auto scores = [&](const char* kst, auto par) {
        f32x16 (&sacc)[T::KB] = sbuf[decltype(par)::value];
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
            sacc[kb] = f32x16{};
#pragma unroll
            for (int s = 0; s < T::KS; ++s) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(kst + kr_off[s] + kb * 32 * T::ROW);
                sacc[kb] = mfma32x32x16(a, qf[s], sacc[kb]);
            }
        }
        // Schedule: each K operand read goes three MFMAs ahead of its use.
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // DS reads
#pragma unroll
        for (int i = 0; i < T::KB * T::KS - 3; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    };

    auto softmax_pv = [&](const int j, const char* vst, auto par, auto masked) {
        // No fusing of a separate multiply and add into one FMA here (the compiler may do it
        // or not depending on the code around): the row sum's rescale-then-add must round
        // the same way in the single-pass kernel and the statistics pass.
#pragma clang fp contract(off)
        f32x16 (&sacc)[T::KB] = sbuf[decltype(par)::value];
        if constexpr (decltype(masked)::value) {
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
        if constexpr (PASS == 1) {
            // Fast path of the statistics pass: the exponentials against the current
            // reference, without the row max. If this lane's share of the row sum grew by
            // at most 128, none of them exceeds ~128 (the sum's rounding hides less than 128
            // while it stays below 2^26), so no score lies more than 8 (log2 units) above
            // the reference: the path below would keep the reference and add the same
            // values in the same order. Otherwise (or while the reference is still -inf)
            // the wave takes that path.
            const float mb0 = m_used * scale_log2;
            float l_new = l_part;
#pragma unroll
            for (int t = 0; t < T::PS; ++t) {
                const int kb = t >> 1, base = (t & 1) * 8;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float p0 = fast_exp2(fmaf(sacc[kb][base + 2 * u], scale_log2, -mb0));
                    const float p1 = fast_exp2(fmaf(sacc[kb][base + 2 * u + 1], scale_log2, -mb0));
                    l_new += p0 + p1;
                }
            }
            const bool ok = m_used != -INFINITY && l_new <= l_part + 128.f;
            if (!__builtin_amdgcn_ballot_w64(!ok)) {
                l_part = l_new;
                return;
            }
        }
        // Every row attends key 0 (causal rows see the whole prefix), so after the first
        // tile the max is finite and no -inf - -inf can occur.
        if constexpr (PASS != 2) {
        float mx = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        mx = fmaxf(mx, xor32(mx));
        const float m_cand = fmaxf(m_used, mx);
        const bool move = m_cand > m_used + tau_raw;
        if (__builtin_amdgcn_ballot_w64(move)) {
            // Only rows whose max moved change their reference (alpha = 1 elsewhere), so
            // a row's arithmetic never depends on the other rows of the wave.
            // A row that does not move keeps alpha = 1 (its reference may still be -inf,
            // where m_used - m_used would be NaN).
            const float m_new = move ? m_cand : m_used;
            const float alpha = move ? fast_exp2((m_used - m_new) * scale_log2) : 1.f;
            m_used = m_new;
            l_part *= alpha;  // the first pass keeps no output to rescale
        }
        }
        const float mb = PASS == 2 ? mb_fixed : m_used * scale_log2;
#pragma unroll
        for (int t = 0; t < T::PS; ++t) {
            const int kb = t >> 1, base = (t & 1) * 8;
            u32x4 pf;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float p0 = fast_exp2(fmaf(sacc[kb][base + 2 * u], scale_log2, -mb));
                const float p1 = fast_exp2(fmaf(sacc[kb][base + 2 * u + 1], scale_log2, -mb));
                pf[u] = pack_bf16x2(p0, p1);
                if constexpr (PASS != 2) l_part += p0 + p1;  // fp32 sum of the unrounded exponentials
            }
            if constexpr (PASS != 1) {
#pragma unroll
                for (int db = 0; db < T::DB; ++db) {
                    // keys 16t + 4g + {0..3} and 16t + 8 + 4g + {0..3} at dim 32db + col
                    const u32x2 a0 = lds_read_tr(vst + vr_off[db] + (t * 16) * T::ROW);
                    const u32x2 a1 = lds_read_tr(vst + vr_off[db] + (t * 16 + 8) * T::ROW);
                    const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
                    oacc[db] = mfma32x32x16(a, pf, oacc[db]);
                }
            }
        }
        if constexpr (PASS != 1) {
            // Schedule: the V^T operand reads go two MFMAs ahead of their use.
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < T::PS * T::DB - 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // Tile j with stage parity par = j & 1: K_j and V_j are in ks<par>, vs<par>.
    auto step = [&](const int j, auto par, auto masked) {
        constexpr int pv = decltype(par)::value;
        using Next = std::integral_constant<int, 1 - pv>;
        char* k_cur = pv ? ks1 : ks0;   // K_j: its stage receives K_{j+2}
        char* k_nxt = pv ? ks0 : ks1;   // K_{j+1}
        char* v_cur = pv ? vs1 : vs0;   // V_j
        char* v_nxt = pv ? vs0 : vs1;   // receives V_{j+1}
        if (j + 2 < n_tiles) load_k(j + 2, k_cur);
        if (PASS != 1 && j + 1 < n_tiles) load_v(j + 1, v_nxt);
        if (j + 1 < n_tiles) scores(k_nxt, Next{});
        softmax_pv(j, v_cur, par, masked);
        __syncthreads();  // completes the loads above and publishes K_{j+2}, V_{j+1}
    };

    // Prologue: K_0, V_0, K_1 in place; S_0 computed; a barrier separates the S_0 reads
    // from step 0's load into K_0's stage.
    load_k(0, ks0);
    if (PASS != 1) load_v(0, vs0);
    if (n_tiles > 1) load_k(1, ks1);
    __syncthreads();
    scores(ks0, P0{});
    __syncthreads();

    // Unmasked tiles two at a time (stage parity alternates), then the rest with masking.
    const int n_plain = min(full, n_tiles);
    int j = 0;
    for (; j + 1 < n_plain; j += 2) {
        step(j, P0{}, std::false_type{});
        step(j + 1, P1{}, std::false_type{});
    }
    for (; j < n_tiles; j += 2) {
        step(j, P0{}, std::true_type{});
        if (j + 1 < n_tiles) step(j + 1, P1{}, std::true_type{});
    }

    // ---- epilogue: the first pass stores lse = M + ln L, the second O (normalised already) ----
    if constexpr (PASS == 1) {
        const float l = l_part + xor32(l_part);
        if (qrow < Nq && g == 0)
            lse[(size_t)pair * Nq + qrow] = (m_used * scale_log2 + fast_log2(l)) * kLn2;
        return;
    }
    if (qrow < Nq) {
        uint16_t* orow = o + ((size_t)pair * Nq + qrow) * D;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d0 = db * 32 + r * 8 + g * 4;
                u32x2 pk = {pack_bf16x2(oacc[db][r * 4 + 0], oacc[db][r * 4 + 1]),
                            pack_bf16x2(oacc[db][r * 4 + 2], oacc[db][r * 4 + 3])};
                *reinterpret_cast<u32x2*>(orow + d0) = pk;
            }
    }
}

template <int D, bool CAUSAL, int PASS>
hipError_t launch_typed(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int Hkv, int Nq, int Nk, float scale, hipStream_t stream) {
    using T = Tile<D>;
    const int n_qt = (Nq + T::BM - 1) / T::BM;
    const int BH = B * H;
    const float scale_log2 = scale * kLog2e;
    const float tau_raw = 8.0f / scale_log2;  // move the reference max past +8 in log2 units
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, PASS>), dim3(n_qt * BH), dim3(T::NT), 0,
                       stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, H, Hkv,
                       Nq, Nk, n_qt, BH, scale_log2, tau_raw);
    return hipGetLastError();
}

}  // namespace

template <int D, bool CAUSAL>
hipError_t launch_two_pass(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int Hkv, int Nq, int Nk, float scale, hipStream_t stream) {
    hipError_t e = launch_typed<D, CAUSAL, 1>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream);
    if (e != hipSuccess) return e;
    return launch_typed<D, CAUSAL, 2>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream);
}

hipError_t launch_fwd_bf16_two_pass(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int B, int H, int Hkv, int Nq, int Nk, int d,
                                    int causal, float scale, hipStream_t stream) {
    if (d == 128)
        return causal ? launch_two_pass<128, true>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream)
                      : launch_two_pass<128, false>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream);
    return causal ? launch_two_pass<64, true>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream)
                  : launch_two_pass<64, false>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream);
}


}  // namespace kvfa
