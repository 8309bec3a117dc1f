// Single-token decode against a paged KV cache: split-K attention + log-sum-exp merge.
//
// Method: glossary entry "KV Cache (Anahtar-Değer Önbelleği)" (yapayzekasozluk.tr,
// tag "Attention"): the new token's query reads the cached K/V of every earlier token
// (its own K/V already appended); the cache lives in fixed-size pages; under GQA
// several query heads share one K/V head. The softmax over the cached keys uses the
// running max / running sum merge of page "Donanıma Duyarlı Algoritma Tasarımı:
// FlashAttention", "Online Softmax Prensibi" steps 1-5, both inside a split (page by
// page) and across splits (the combine kernel merges (O_k, lse_k) pairs, the same
// algebra expressed through one log-sum-exp per part).
//
// gfx950 mapping (this design):
// * Work-group = (sequence, KV head, split of `split_tokens` keys), 4 waves; wave w
//   takes pages w, w+4, ... of its split. All query heads of the GQA group are
//   served from one read of each K/V page, so every cached byte is read once.
// * Scores: S^T[token][head] = K_page Q^T with v_mfma_f32_16x16x32_bf16 — one page
//   (16 tokens) is exactly the MFMA's 16 rows, the group's heads fill its columns.
//   The MFMA wants one token per lane of a 16-lane group, HBM wants whole rows per
//   16 lanes: K pages therefore go HBM -> LDS by direct loads (buffer_load ... lds, each
//   instruction 1 KiB of whole rows, 16-byte chunks XOR-swizzled by row) into a
//   per-wave double buffer, and the A operand is read from there without bank
//   conflicts.
// * P.V: plain FMAs. A lane owns one 16-byte chunk of V rows (8 dims) for a subset of
//   the page's tokens and accumulates all heads of the group; the probabilities reach
//   it through a small per-wave LDS table.
// * The split's partial result (normalised O_k, lse_k in log2 units) goes to the
//   caller's workspace; a second kernel merges the splits in order.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace kvfa {

namespace {

constexpr int kPage = 16;
constexpr int kWaves = 4;

// FP8 = true: the cache holds e4m3 bytes with one scale per KV head for K and one for V
// (dequantised value = byte value x scale). K bytes are converted exactly to bf16 for the
// MFMA and V bytes to fp32 for the P.V FMAs; the K scale is folded into the softmax
// scale and the V scale is applied to the split's output, so the arithmetic is that of
// the dequantised cache. Each cached token costs half the bytes of the bf16 cache.
template <int D, int GH, bool FP8>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kcache,
    const void* __restrict__ vcache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, float* __restrict__ o_part,
    float* __restrict__ lse_part, int H, int Hkv, int g, int n_hg, int num_pages,
    int max_pages, int max_seq_len, int split_tokens, int max_splits, float scale_log2_in,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
    constexpr int ES = FP8 ? 1 : 2;    // bytes per cached element
    using KVec = std::conditional_t<FP8, u32x2, u32x4>;  // 8 cached elements
    constexpr int CH = D / 8;          // 16-byte chunks per token row
    constexpr int TG = 64 / CH;        // token groups of the P.V lane layout
    constexpr int TPL = kPage / TG;    // tokens per lane in P.V
    constexpr int KS = D / 32;         // MFMA k-steps over the head dimension
    constexpr int ROWB = D * ES;       // bytes of one cached row (token, KV head)
    constexpr int KCH = ROWB / 16;     // 16-byte chunks per row
    constexpr int PAGEB = kPage * ROWB;            // bytes of one page's K rows
    constexpr int KDMA = PAGEB / 1024;             // 1 KiB direct loads per page
    static_assert(KDMA >= 1 && KDMA * 1024 == PAGEB, "whole 1 KiB loads per page");
    // Per wave: two K stages (separate arrays, so the compiler can tell a read of one from
    // the direct loads into the other); after the wave's loop its partial output for the
    // cross-wave merge reuses the first stage when it fits.
    __shared__ __attribute__((aligned(1024))) char kst_a[kWaves][PAGEB];
    __shared__ __attribute__((aligned(1024))) char kst_b[kWaves][PAGEB];
    constexpr bool RO_IN_A = GH * D * 4 <= PAGEB;
    __shared__ float red_o_x[RO_IN_A ? 1 : kWaves * GH * D];
    auto red_o = [&](int ww) -> float* {  // [GH][D] of wave ww
        if constexpr (RO_IN_A) return reinterpret_cast<float*>(kst_a[ww]);
        else return red_o_x + ww * GH * D;
    };
    __shared__ float p_lds[kWaves][kPage][GH];
    __shared__ float a_lds[kWaves][GH];
    __shared__ float red_m[kWaves][GH];
    __shared__ float red_l[kWaves][GH];

    const int s = blockIdx.z;
    const int kvh = blockIdx.x / n_hg, hg = blockIdx.x % n_hg;
    const int split = blockIdx.y;
    const int L = min(max(seq_lens[s], 0), max_seq_len);
    const int t0 = split * split_tokens;
    if (t0 >= L) return;  // uniform: this split holds no cached token
    const int t1 = min(t0 + split_tokens, L);
    const int first_page = t0 / kPage;
    const int n_pg = (t1 - t0 + kPage - 1) / kPage;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
    const int n = lane & 15;     // head column of S^T held by this lane
    const int kq = lane >> 4;    // k-slot group / token quad of S^T
    const int tg = lane / CH, c = lane % CH;  // P.V layout: token group, V chunk
    const int h0 = kvh * g + hg * GH;
    const int nheads = min(GH, g - hg * GH);
    const size_t tok_stride = (size_t)Hkv * D;  // elements between consecutive slots
    // Softmax scale in log2 units (times the K scale for an fp8 cache) and the V scale.
    float scale_log2 = scale_log2_in, v_sc = 1.f;
    if constexpr (FP8) {
        scale_log2 *= k_scale[kvh];
        v_sc = v_scale[kvh];
    }
    // Move the reference max past +8 in log2 units (with a zero K scale every score is 0:
    // the first page then moves the reference and every later one keeps it).
    const float tau_raw = scale_log2 > 0.f ? 8.0f / scale_log2 : 0.f;

    // B operand (Q^T): Q[s][h0+n][8*(4j + kq) .. +7], zero for padding columns.
    u32x4 qf[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        qf[j] = u32x4{0, 0, 0, 0};
        if (n < nheads)
            qf[j] = *reinterpret_cast<const u32x4*>(q + ((size_t)s * H + h0 + n) * D +
                                                     (j * 4 + kq) * 8);
    }

    float m_used = -INFINITY, l_part = 0.f;
    float oacc[GH][8];
#pragma unroll
    for (int hh = 0; hh < GH; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[hh][e] = 0.f;

    // This wave's pages are first_page + w + kWaves*i, i < n_my. Lane i holds the
    // physical id of the i-th one, so no page-table load sits on the loop's critical path.
    const int n_my = w < n_pg ? (n_pg - w + kWaves - 1) / kWaves : 0;
    int pid_lane = -1;
    if (lane < n_my) pid_lane = page_table[(size_t)s * max_pages + first_page + w + kWaves * lane];
    // Let the ids arrive once, here; afterwards the register no longer counts as a pending
    // load, so reading it inside the loop does not wait for the page loads in flight.
    __asm__ volatile("" : "+v"(pid_lane));

    // Issue the loads of the wave's it-th page (K rows as the MFMA A operand, V chunks for
    // the P.V lanes). Returns false for an out-of-range page id, which is never read.
    // Loads are issued unconditionally (a zero-size descriptor for an invalid page id
    // makes them return zeros without touching memory), so the wait counts stay exact.
    // The cache is read once per call: the loads carry the nontemporal hint.
    const uint32_t span = (uint32_t)((kPage - 1) * tok_stride + D) * ES;
    const uint32_t v_off = (uint32_t)(tg * tok_stride + c * 8) * ES;
    // K direct loads: lane L of the i-th 1 KiB piece fills stage byte 1024 i + 16 L, i.e.
    // row r, physical chunk pc, with logical chunk pc ^ (r % KCH) of cached row r.
    uint32_t kd_off[KDMA];
#pragma unroll
    for (int i = 0; i < KDMA; ++i) {
        const int byte = 1024 * i + 16 * lane;
        const int r = byte / ROWB, pc = (byte % ROWB) / 16;
        kd_off[i] = (uint32_t)(r * tok_stride * ES + ((pc ^ (r % KCH)) * 16));
    }
    // A operand of k-step j: token n, elements 32 j + 8 kq .. +7 (8 ES bytes).
    int kr_off[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int b = (32 * j + 8 * kq) * ES;
        kr_off[j] = n * ROWB + (((b / 16) ^ (n % KCH)) * 16) + b % 16;
    }
    char* const kst0 = kst_a[w];
    char* const kst1 = kst_b[w];
    auto load8 = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) -> KVec {
        if constexpr (FP8) return buf_load8_nt(r, off);
        else return buf_load16_nt(r, off);
    };
    auto load_page = [&](int it, char* kst, KVec (&vv)[TPL]) -> bool {
        const int pid = __builtin_amdgcn_readlane(pid_lane, it);
        const bool valid = (unsigned)pid < (unsigned)num_pages;
        const size_t page_base = (size_t)(valid ? pid : 0) * kPage * tok_stride + (size_t)kvh * D;
        const auto rk = make_rsrc(static_cast<const char*>(kcache) + page_base * ES, valid ? span : 0u);
        const auto rv = make_rsrc(static_cast<const char*>(vcache) + page_base * ES, valid ? span : 0u);
#pragma unroll
        for (int i = 0; i < KDMA; ++i) buf_load16_lds_nt(rk, kst + 1024 * i, kd_off[i], 0u);
#pragma unroll
        for (int i = 0; i < TPL; ++i)
            vv[i] = load8(rv, v_off + (uint32_t)(TG * i * tok_stride) * ES);
        return valid;
    };

    KVec vA[TPL], vB[TPL];
    bool okA = load_page(0, kst0, vA);   // a lane past the wave's pages holds id -1
    bool okB = false;
    // Every load of the page before this one's successor has landed: its K rows in LDS
    // (direct loads are counted by vmcnt only) and its V registers.
    auto wait_page = [&]() __attribute__((always_inline)) {
        constexpr int later = KDMA + TPL;  // loads of the page issued after it
        static_assert(later < 64, "vmcnt field");
        __builtin_amdgcn_s_waitcnt((later & 15) | ((later >> 4) << 14) | (7 << 4) | (15 << 8));
    };
    auto page_compute = [&](const char* KST, const KVec (&VV)[TPL], const bool OK, const int IT) {
        if (OK) {
            const int tok0 = (first_page + w + kWaves * IT) * kPage;
            KVec KF[KS];
#pragma unroll
            for (int j = 0; j < KS; ++j) KF[j] = *reinterpret_cast<const KVec*>(KST + kr_off[j]);

            // S^T: acc[i] = score of token 4*kq + i for head column n
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                if constexpr (FP8) {
                    const u32x2 lo = fp8x4_to_bf16x4(KF[j][0]), hi = fp8x4_to_bf16x4(KF[j][1]);
                    acc = mfma16x16x32(u32x4{lo[0], lo[1], hi[0], hi[1]}, qf[j], acc);
                } else {
                    acc = mfma16x16x32(KF[j], qf[j], acc);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tok0 + kq * 4 + i >= t1) acc[i] = -INFINITY;

            float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float m_cand = fmaxf(m_used, mx);  // finite: a page's first token is valid
            const bool move = m_cand > m_used + tau_raw;
            const bool resc = __builtin_amdgcn_ballot_w64(move) != 0;
            if (resc) {
                const float m_new = move ? m_cand : m_used;  // alpha = 1 for unmoved heads
                const float alpha = move ? fast_exp2((m_used - m_new) * scale_log2) : 1.f;
                m_used = m_new;
                l_part *= alpha;
                if (kq == 0 && n < GH) a_lds[w][n] = alpha;
            }
            const float mb = m_used * scale_log2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(fmaf(acc[i], scale_log2, -mb));
                l_part += p;
                if (n < GH) p_lds[w][kq * 4 + i][n] = p;
            }
            wave_lds_fence();

            if (resc) {
#pragma unroll
                for (int hh = 0; hh < GH; ++hh) {
                    const float a = a_lds[w][hh];
#pragma unroll
                    for (int e = 0; e < 8; ++e) oacc[hh][e] *= a;
                }
            }
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const int tl = tg + TG * i;
                const bool ok = tok0 + tl < t1;  // slots past the sequence may hold anything
                float x[8];
                if constexpr (FP8) {
                    fp8x4_to_f32x4(ok ? VV[i][0] : 0u, x);
                    fp8x4_to_f32x4(ok ? VV[i][1] : 0u, x + 4);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t wd = ok ? VV[i][e] : 0u;
                        x[2 * e] = bf16lo(wd);
                        x[2 * e + 1] = bf16hi(wd);
                    }
                }
#pragma unroll
                for (int hh = 0; hh < GH; ++hh) {
                    const float p = p_lds[w][tl][hh];
#pragma unroll
                    for (int e = 0; e < 8; ++e) oacc[hh][e] = fmaf(p, x[e], oacc[hh][e]);
                }
            }
            wave_lds_fence();
        }
    };
    for (int it = 0; it < n_my; it += 2) {
        okB = load_page(it + 1, kst1, vB);
        wait_page();
        page_compute(kst0, vA, okA, it);
        okA = load_page(it + 2, kst0, vA);
        wait_page();
        page_compute(kst1, vB, okB, it + 1);
    }
    // The loop ends with two pages' loads still in flight (past the wave's last page: zero
    // descriptors, but their LDS writes land in the stages reused below).
    __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));

    // ---- reduce within the wave, then across the 4 waves ----
    float l = l_part;
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
#pragma unroll
    for (int hh = 0; hh < GH; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = oacc[hh][e];
#pragma unroll
            for (int msk = CH; msk < 64; msk <<= 1) x += shfl_xor(x, msk);
            oacc[hh][e] = x;
        }
    if (kq == 0 && n < GH) {
        red_m[w][n] = m_used;
        red_l[w][n] = l;
    }
    if (tg == 0) {
        float* ro = red_o(w);
#pragma unroll
        for (int hh = 0; hh < GH; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) ro[hh * D + c * 8 + e] = oacc[hh][e];
    }
    __syncthreads();

    for (int idx = tid; idx < nheads * D; idx += 256) {
        const int hh = idx / D, dd = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_m[ww][hh]);
        float lsum = 0.f, acc = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                const float mw = red_m[ww][hh];  // -inf for a wave that saw no token
                const float f = mw == -INFINITY ? 0.f : fast_exp2((mw - M) * scale_log2);
                lsum = fmaf(f, red_l[ww][hh], lsum);
                acc = fmaf(f, red_o(ww)[hh * D + dd], acc);
            }
        }
        const size_t row = ((size_t)s * H + h0 + hh) * max_splits + split;
        o_part[row * D + dd] = M != -INFINITY ? acc / lsum * v_sc : 0.f;
        if (dd == 0)
            lse_part[row] = M != -INFINITY ? M * scale_log2 + fast_log2(lsum) : -INFINITY;
    }
}

// Merge the splits of each (sequence, head): LSE = log2 sum_k 2^lse_k (relative to the
// largest), O = sum_k 2^(lse_k - LSE) O_k. One wave per (sequence, head), kCombineHeads
// heads per work-group. The split statistics are spread over the lanes (one split per
// lane, wave reductions for the max and the sum); each lane then owns D/64 output dims and
// walks the splits with eight partial rows in flight, the weights broadcast from the lane
// that holds them.
constexpr int kCombineHeads = 4;
template <int D>
__global__ __launch_bounds__(64 * kCombineHeads) void decode_combine_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ o, float* __restrict__ lse,
    int H, int max_seq_len, int split_tokens, int max_splits) {
    constexpr int PER = D / 64;  // output dims per lane (2 or 1)
    const int s = blockIdx.y, lane = threadIdx.x & 63;
    const int h = blockIdx.x * kCombineHeads + (threadIdx.x >> 6);
    if (h >= H) return;  // uniform per wave
    const int L = min(max(seq_lens[s], 0), max_seq_len);
    const int ns = (L + split_tokens - 1) / split_tokens;
    const size_t row = (size_t)s * H + h;
    const float* lp = lse_part + row * max_splits;
    const float* op = o_part + row * max_splits * D + lane * PER;

    float m = -INFINITY;
    for (int k = lane; k < ns; k += 64) m = fmaxf(m, lp[k]);
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) m = fmaxf(m, shfl_xor(m, msk));
    const float M = m;  // -inf: no split holds a token (L = 0)

    float out[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = 0.f;
    float wsum = 0.f;
    if (M != -INFINITY) {
        for (int kb = 0; kb < ns; kb += 64) {
            // weight of split kb + lane (0 past the last split)
            const float fl = kb + lane < ns ? fast_exp2(lp[kb + lane] - M) : 0.f;
            wsum += fl;
            const int cnt = min(64, ns - kb);
            auto fw = [&](int kk) {
                return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), kk));
            };
            int kk = 0;
            for (; kk + 8 <= cnt; kk += 8) {
                float x[8][PER];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float* src = op + (size_t)(kb + kk + u) * D;
                    if constexpr (PER == 2) {
                        const f32x2 v2 = *reinterpret_cast<const f32x2*>(src);
                        x[u][0] = v2[0];
                        x[u][1] = v2[1];
                    } else {
                        x[u][0] = src[0];
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float f = fw(kk + u);
#pragma unroll
                    for (int e = 0; e < PER; ++e) out[e] = fmaf(f, x[u][e], out[e]);
                }
            }
            for (; kk < cnt; ++kk) {
                const float f = fw(kk);
                const float* src = op + (size_t)(kb + kk) * D;
#pragma unroll
                for (int e = 0; e < PER; ++e) out[e] = fmaf(f, src[e], out[e]);
            }
        }
#pragma unroll
        for (int msk = 1; msk < 64; msk <<= 1) wsum += shfl_xor(wsum, msk);
        const float inv = 1.f / wsum;
#pragma unroll
        for (int e = 0; e < PER; ++e) out[e] *= inv;
    }
    uint16_t* orow = o + row * D + lane * PER;
    if constexpr (PER == 2) {
        *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(out[0], out[1]);
    } else {
        orow[0] = (uint16_t)(pack_bf16x2(out[0], 0.f) & 0xffffu);
    }
    if (lse != nullptr && lane == 0)
        lse[row] = M != -INFINITY ? (M + fast_log2(wsum)) * kLn2 : -INFINITY;
}

template <int D, int GH, bool FP8>
hipError_t launch_split(const void* q, const void* kc, const void* vc, const int32_t* pt,
                        const int32_t* sl, float* o_part, float* lse_part, int num_seqs, int H,
                        int Hkv, int g, int n_hg, int num_pages, int max_pages, int max_seq_len,
                        int split_tokens, int max_splits, float scale, const float* k_scale,
                        const float* v_scale, hipStream_t stream) {
    const float scale_log2 = scale * kLog2e;
    // KV heads vary fastest: the work-groups covering one token range of one sequence
    // are dispatched together, so each physical page (all KV heads of 16 slots, contiguous)
    // is read by concurrently running work-groups.
    dim3 grid(Hkv * n_hg, max_splits, num_seqs);
    hipLaunchKernelGGL((decode_split_kernel<D, GH, FP8>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), kc, vc, pt, sl, o_part, lse_part, H, Hkv,
                       g, n_hg, num_pages, max_pages, max_seq_len, split_tokens, max_splits,
                       scale_log2, k_scale, v_scale);
    return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_split_d(int GH, const void* q, const void* kc, const void* vc,
                          const int32_t* pt, const int32_t* sl, float* o_part, float* lse_part,
                          int num_seqs, int H, int Hkv, int g, int n_hg, int num_pages,
                          int max_pages, int max_seq_len, int split_tokens, int max_splits,
                          float scale, const float* ks, const float* vs, hipStream_t stream) {
    if (GH == 4)
        return launch_split<D, 4, FP8>(q, kc, vc, pt, sl, o_part, lse_part, num_seqs, H, Hkv, g,
                                       n_hg, num_pages, max_pages, max_seq_len, split_tokens,
                                       max_splits, scale, ks, vs, stream);
    if (GH == 8)
        return launch_split<D, 8, FP8>(q, kc, vc, pt, sl, o_part, lse_part, num_seqs, H, Hkv, g,
                                       n_hg, num_pages, max_pages, max_seq_len, split_tokens,
                                       max_splits, scale, ks, vs, stream);
    return launch_split<D, 16, FP8>(q, kc, vc, pt, sl, o_part, lse_part, num_seqs, H, Hkv, g,
                                    n_hg, num_pages, max_pages, max_seq_len, split_tokens,
                                    max_splits, scale, ks, vs, stream);
}

}  // namespace

int decode_split_tokens(int num_seqs, int Hkv, int max_seq_len, int page_size) {
    // A work-group has a fixed cost (page ids, first loads, merging its waves, writing
    // its partial result) and the last round of work-groups leaves CUs idle. Splits of 512
    // tokens are lengthened (in steps of 128) while the launch would exceed about six
    // rounds of resident work-groups (256 CUs x 4), and shortened when fewer than 2048
    // work-groups would be launched. (T <= 2048 keeps every wave's page count, plus the
    // two pages it prefetches past its last one, within the 64 lanes that hold its page
    // ids.)
    constexpr long long kResident = 256 * 4;
    auto wgs = [&](int T) { return (long long)num_seqs * Hkv * ((max_seq_len + T - 1) / T); };
    int T = 512;
    while (T < 2048 && wgs(T) > 6 * kResident) T += 128;
    while (T > 64 && wgs(T) < 2048) T >>= 1;
    if (T < page_size) T = page_size;
    return T;
}

size_t decode_workspace_bytes(int num_seqs, int H, int Hkv, int d, int max_seq_len,
                              int page_size) {
    const int T = decode_split_tokens(num_seqs, Hkv, max_seq_len, page_size);
    const size_t max_splits = (size_t)(max_seq_len + T - 1) / T;
    const size_t rows = (size_t)num_seqs * H * max_splits;
    return rows * (size_t)d * sizeof(float) + rows * sizeof(float);
}

hipError_t launch_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* page_table, const int32_t* seq_lens, void* o,
                               float* lse, int num_seqs, int H, int Hkv, int d, int num_pages,
                               int max_pages_per_seq, int max_seq_len, float scale,
                               void* workspace, hipStream_t stream, const float* k_scale,
                               const float* v_scale) {
    const bool fp8 = k_scale != nullptr;
    const int T = decode_split_tokens(num_seqs, Hkv, max_seq_len, kPage);
    const int max_splits = (max_seq_len + T - 1) / T;
    const int g = H / Hkv;
    const int GH = g <= 4 ? 4 : g <= 8 ? 8 : 16;
    const int n_hg = g <= 16 ? 1 : g / 16;
    float* o_part = static_cast<float*>(workspace);
    float* lse_part = o_part + (size_t)num_seqs * H * max_splits * d;

    hipError_t e;
    if (d == 128)
        e = fp8 ? launch_split_d<128, true>(GH, q, k_cache, v_cache, page_table, seq_lens, o_part,
                                            lse_part, num_seqs, H, Hkv, g, n_hg, num_pages,
                                            max_pages_per_seq, max_seq_len, T, max_splits, scale,
                                            k_scale, v_scale, stream)
                : launch_split_d<128, false>(GH, q, k_cache, v_cache, page_table, seq_lens,
                                             o_part, lse_part, num_seqs, H, Hkv, g, n_hg,
                                             num_pages, max_pages_per_seq, max_seq_len, T,
                                             max_splits, scale, nullptr, nullptr, stream);
    else
        e = fp8 ? launch_split_d<64, true>(GH, q, k_cache, v_cache, page_table, seq_lens, o_part,
                                           lse_part, num_seqs, H, Hkv, g, n_hg, num_pages,
                                           max_pages_per_seq, max_seq_len, T, max_splits, scale,
                                           k_scale, v_scale, stream)
                : launch_split_d<64, false>(GH, q, k_cache, v_cache, page_table, seq_lens,
                                            o_part, lse_part, num_seqs, H, Hkv, g, n_hg,
                                            num_pages, max_pages_per_seq, max_seq_len, T,
                                            max_splits, scale, nullptr, nullptr, stream);
    if (e != hipSuccess) return e;
    dim3 grid((H + kCombineHeads - 1) / kCombineHeads, num_seqs);
    if (d == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, grid, dim3(64 * kCombineHeads), 0, stream,
                           o_part, lse_part, seq_lens, static_cast<uint16_t*>(o), lse, H,
                           max_seq_len, T, max_splits);
    else
        hipLaunchKernelGGL(decode_combine_kernel<64>, grid, dim3(64 * kCombineHeads), 0, stream,
                           o_part, lse_part, seq_lens, static_cast<uint16_t*>(o), lse, H,
                           max_seq_len, T, max_splits);
    return hipGetLastError();
}

}  // namespace kvfa
