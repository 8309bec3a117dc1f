// bf16 exact attention (prefill) for launches too small to fill the chip: each work-group
// owns 32 query rows of one (batch, head), and its four waves split that tile's keys.
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
// fewer of them than compute units the launch lasts as long as the longest sweep, not as
// long as the chip needs for the work (B2 H8 N1024 d64 causal: 64 work-groups, each up
// to 16 tiles of 64 keys one after the other). Here the longest chain is a quarter of
// that and there are 8x as many work-groups.
//
// gfx950 mapping:
// * 256 threads = 4 waves; wave w takes key tiles w, w + 4, w + 8, ... of its row block.
//   The waves never wait for each other until the merge.
// * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with the wave's 32 Q rows held as B
//   operands; each lane owns one query column, so the row max is in-lane plus one
//   exchange with lane ^ 32. K operands are loaded from memory straight into registers
//   in the MFMA's layout (a lane reads 16 contiguous bytes of one key row), one tile
//   ahead of use.
// * O^T += V^T P^T: V tiles go from memory straight into LDS (buffer_load ... lds), two
//   stages per wave, two tiles ahead, and are read back through transposing LDS reads
//   (ds_read_b64_tr_b16), 16-byte chunks XOR-swizzled by row so those reads are
//   conflict-free.
// * Merge: every wave writes its (m, l) per row and its fp32 output accumulator to LDS
//   over its own V stages; after a work-group barrier wave w combines rows' dims
//   32 db + 8 w + {0..7} of all four parts and stores them as bf16, and wave 0 stores
//   lse = m + ln l.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "prefill_common.h"

namespace kvfa {

namespace {
using namespace prefill;

template <int D>
struct TileKS {
    static constexpr int NW = 4;                 // waves per work-group (key parts)
    static constexpr int NT = 64 * NW;           // threads per work-group
    static constexpr int BM = 32;                // query rows per work-group
    static constexpr int BN = D == 64 ? 64 : 32; // keys per tile
    static constexpr int KB = BN / 32;           // 32-key blocks of S^T
    static constexpr int KS = D / 16;            // MFMA k-steps of Q.K (16 dims each)
    static constexpr int DB = D / 32;            // 32-dim blocks of O^T
    static constexpr int PS = BN / 16;           // MFMA k-steps of P.V (16 keys each)
    static constexpr int ROW = D * 2;            // bytes per K/V row
    static constexpr int TILE = BN * ROW;        // bytes of one V tile
    static constexpr int DMA = TILE / 1024;      // 1 KiB direct loads per V tile (one wave)
    static constexpr int KL = KB * KS;           // 16-byte K loads per lane per tile
    static constexpr int PART = DB * 16 * 64 * 4;  // bytes of one wave's fp32 accumulator
    static_assert(DMA * 1024 == TILE && PART <= 2 * TILE, "merge area fits in the V stages");
    static_assert(PART % 1024 == 0, "whole 1 KiB chunks");
    static_assert(2 * KL + DMA < 64, "vmcnt field");
};

// Waits until at most n vector-memory loads of this wave are in flight (n constant).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Waits until every LDS read of this wave has returned. A direct load into an LDS stage
// must not be issued before the reads of the stage's previous tile are done: the hardware
// does not order a read still in the LDS queue before a later load's write to the same
// bytes, and the compiler may interleave the load with the reads' MFMAs.
__device__ __forceinline__ void wait_lds_reads() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_ks_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                   float* __restrict__ lse, int H, int Hkv, int Nq, int Nk, int n_qt, int BH,
                   float scale_log2, float tau_raw) {
    using T = TileKS<D>;
    constexpr int BN = T::BN;
    // V stages of wave w: vs0[w], vs1[w] (separate arrays, so the compiler can tell a load
    // into one stage from reads of the other); reused for the merge.
    __shared__ __attribute__((aligned(1024))) char vs0[T::NW][T::TILE];
    __shared__ __attribute__((aligned(1024))) char vs1[T::NW][T::TILE];
    __shared__ float red[T::NW][2][32];  // per wave: m (log2 units) and l of each row

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;  // query row (column of S^T) owned by this lane
    const int g = lane >> 5;    // which half of the MFMA k-slots this lane supplies

    int pair, qt;
    map_work(blockIdx.x, n_qt, BH, H / Hkv, CAUSAL, pair, qt);
    const int b = pair / H, h = pair % H;
    const int kvh = h / (H / Hkv);
    const int q0 = qt * T::BM;
    const int off = Nk - Nq;
    const int qrow = q0 + col;

    const auto rq = make_rsrc(q + (size_t)pair * Nq * D, (uint32_t)Nq * D * 2);
    const auto rk = make_rsrc(k + ((size_t)b * Hkv + kvh) * Nk * D, (uint32_t)Nk * D * 2);
    const auto rv = make_rsrc(v + ((size_t)b * Hkv + kvh) * Nk * D, (uint32_t)Nk * D * 2);
    // Zero-size descriptors for the loads of tiles past the row block's last one: they still
    // count as issued loads (the waits keep fixed counts) but fetch nothing.
    const auto rk_none = make_rsrc(k, 0u);
    const auto rv_none = make_rsrc(v, 0u);

    // Key tiles of the row block, and the first one that needs a mask.
    const int n_all = (Nk + BN - 1) / BN;
    int n_tiles = n_all, full = Nk / BN;
    if (CAUSAL) {
        const int last_row = min(q0 + T::BM, Nq) - 1;
        n_tiles = min(n_all, (last_row + off) / BN + 1);
        full = min(full, (q0 + off + 1) / BN);
    }
    // This wave's tiles: j_i = w + 4 i, i < n_my.
    const int n_my = w < n_tiles ? (n_tiles - w + T::NW - 1) / T::NW : 0;

    // B operand of S^T = K Q^T: Q[qrow][16 s + 8 g .. +7]; rows past Nq load as zero.
    u32x4 qf[T::KS];
#pragma unroll
    for (int s = 0; s < T::KS; ++s)
        qf[s] = buf_load16(rq, (uint32_t)(qrow * D + s * 16 + g * 8) * 2);

    // K operand (kb, s) of tile j: K[j BN + 32 kb + col][16 s + 8 g .. +7]; the tile's
    // offset is uniform (a scalar register), the rest a per-lane base plus a constant.
    u32x4 kf[T::KB][T::KS];
    const uint32_t k_lane = (uint32_t)(col * D * 2 + g * 16);
    auto load_k = [&](int j) {
        const auto r = j < n_tiles ? rk : rk_none;
        const uint32_t tile_off = (uint32_t)j * (uint32_t)T::TILE;
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
            for (int s = 0; s < T::KS; ++s)
                kf[kb][s] = __builtin_amdgcn_raw_buffer_load_b128(
                    r, k_lane + (uint32_t)(kb * 32 * D * 2 + s * 32), tile_off, 0);
    };
    // V tile j into one stage: the i-th 1 KiB piece covers tile bytes [1024 i, +1024);
    // lane L fills byte 16 L of it, i.e. row r, physical chunk pc, with logical chunk
    // pc ^ v_swz(r) of row r.
    uint32_t dv_off[T::DMA];
#pragma unroll
    for (int i = 0; i < T::DMA; ++i) {
        const int byte = 1024 * i + 16 * lane;
        const int r = byte / T::ROW, pc = (byte % T::ROW) / 16;
        dv_off[i] = (uint32_t)(r * T::ROW + ((pc ^ v_swz<D>(r)) * 16));
    }
    auto load_v = [&](int j, char* dst) {
        const auto r = j < n_tiles ? rv : rv_none;
#pragma unroll
        for (int i = 0; i < T::DMA; ++i)
            buf_load16_lds(r, dst + 1024 * i, dv_off[i], (uint32_t)j * (uint32_t)T::TILE);
    };
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

    // One tile: scores, mask (tiles from `full` on), running max, exponentials, P.V. Its V
    // is in stage vst. One body serves masked and unmasked tiles (a copy of each made the
    // compiler keep two register assignments live and spill).
    // The loads of the tiles after it are issued whether or not those tiles exist (through
    // zero-size descriptors when they do not: nothing is fetched), so every wait below has
    // one fixed count.
    auto tile = [&](const int j, const char* vst) {
        f32x16 sacc[T::KB];
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
            sacc[kb] = f32x16{};
#pragma unroll
            for (int s = 0; s < T::KS; ++s)
                sacc[kb] = mfma32x32x16(kf[kb][s], qf[s], sacc[kb]);
        }
        load_k(j + T::NW);  // the registers are free once the MFMAs have read them
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
        // V_j has landed once at most the loads issued after it are in flight: K_j, V_{j+4}
        // and K_{j+4}.
        wait_vm<2 * T::KL + T::DMA>();
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
                // keys 16t + 4g + {0..3} and 16t + 8 + 4g + {0..3} at dim 32db + col
                const u32x2 a0 = lds_read_tr(vst + vr_off[db] + (t * 16) * T::ROW);
                const u32x2 a1 = lds_read_tr(vst + vr_off[db] + (t * 16 + 8) * T::ROW);
                const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
                oacc[db] = mfma32x32x16(a, pf, oacc[db]);
            }
        }
    };

    // Issue order V_0, K_0, V_1, then per tile i: K_{i+1} after its scores, V_{i+2} after
    // its P.V, so V_i always has K_i, V_{i+1}, K_{i+1} behind it. Tiles go in pairs (one
    // per stage); with an odd count the pair's second tile does not exist and only its
    // K load is issued, so that the loads stay in the same order on both paths.
    char* st0 = vs0[w];
    char* st1 = vs1[w];
    if (n_my > 0) {
        load_v(w, st0);
        load_k(w);
        load_v(w + T::NW, st1);
        for (int i = 0; i < n_my; i += 2) {
            const int j = w + T::NW * i;
            tile(j, st0);
            wait_lds_reads();
            load_v(j + 2 * T::NW, st0);
            const int j1 = j + T::NW;
            if (i + 1 < n_my) {
                tile(j1, st1);
            } else {
                load_k(j1 + T::NW);
            }
            wait_lds_reads();
            load_v(j1 + 2 * T::NW, st1);
        }
        wait_vm<0>();  // the loads of the tiles past the end land before the stages are reused
    }

    // ---- merge the four parts ----
    // Every load of this wave has landed, so its V stages are free. Accumulator elements
    // (db, 4 r .. 4 r + 3) of all 64 lanes form the 1 KiB chunk c = 4 db + r of wave x's
    // merge area: chunk c of vs0[x], then of vs1[x].
    constexpr int CPS = T::TILE / 1024;  // chunks per stage
    auto chunk = [&](int x, int c) -> char* {
        return c < CPS ? vs0[x] + 1024 * c : vs1[x] + 1024 * (c - CPS);
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
            *reinterpret_cast<f32x4*>(chunk(w, 4 * db + r) + 16 * lane) =
                f32x4{oacc[db][4 * r], oacc[db][4 * r + 1], oacc[db][4 * r + 2], oacc[db][4 * r + 3]};
    __syncthreads();

    // Every row attends key 0, which is in wave 0's first tile, so M is finite.
    float mw[T::NW], M = -INFINITY;
#pragma unroll
    for (int x = 0; x < T::NW; ++x) {
        mw[x] = red[x][0][col];
        M = fmaxf(M, mw[x]);
    }
    float a[T::NW], L = 0.f;
#pragma unroll
    for (int x = 0; x < T::NW; ++x) {
        a[x] = fast_exp2(mw[x] - M);  // 0 for a part that saw no key of the row
        L += a[x] * red[x][1][col];
    }
    const float inv = 1.f / L;
    if (qrow < Nq) {
        uint16_t* orow = o + ((size_t)pair * Nq + qrow) * D;
        const int r = w;  // this wave stores dims 32 db + 8 w + 4 g .. +3
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < T::NW; ++x) {
                const f32x4 p = *reinterpret_cast<const f32x4*>(chunk(x, 4 * db + r) + 16 * lane);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = fmaf(a[x], p[c], acc[c]);
            }
            const u32x2 pk = {pack_bf16x2(acc[0] * inv, acc[1] * inv),
                              pack_bf16x2(acc[2] * inv, acc[3] * inv)};
            *reinterpret_cast<u32x2*>(orow + db * 32 + r * 8 + g * 4) = pk;
        }
        if (lse != nullptr && w == 0 && g == 0)
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
