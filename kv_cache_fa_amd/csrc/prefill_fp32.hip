// fp32 exact attention (prefill), tiled with an online softmax, fp32 arithmetic only.
//
// Method: page "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention". K/V tiles are
// staged in LDS ("FlashAttention'ın Temelleri": blocks in fast on-chip memory); each
// query row keeps a running max m and sum l, merged tile by tile as in "Online
// Softmax Prensibi" steps 1-5, and its output accumulator is rescaled by the same
// exp(m_old - m_new) factor as l so one pass suffices. Work is split over query
// rows ("FlashAttention-2: Optimizasyonlar ve İyileştirmeler", item 1).
//
// Layout: one thread owns one query row (q and the accumulator live in registers);
// a work-group of 64 threads owns 64 consecutive rows of one (batch, head) and walks
// the key tiles in order. exp is the accurate expf of the device math library, not
// the hardware exp2 approximation, so the path stays within fp32 rounding.
#include "common.h"
#include "launch.h"

namespace kvfa {

namespace {

constexpr int kRows = 64;   // query rows per work-group (one per thread)
constexpr int kTile = 32;   // keys per LDS tile

template <int D>
__global__ __launch_bounds__(kRows) void fwd_fp32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int H, int Hkv, int Nq, int Nk,
    int causal, float scale) {
    __shared__ float ks[kTile][D];
    __shared__ float vs[kTile][D];

    const int tid = threadIdx.x;
    const int b = blockIdx.z, h = blockIdx.y;
    const int kvh = h / (H / Hkv);
    const int row = blockIdx.x * kRows + tid;
    const int off = Nk - Nq;  // bottom-right causal alignment

    const float* qh = q + ((size_t)b * H + h) * (size_t)Nq * D;
    const float* kh = k + ((size_t)b * Hkv + kvh) * (size_t)Nk * D;
    const float* vh = v + ((size_t)b * Hkv + kvh) * (size_t)Nk * D;

    float qr[D], acc[D];
    const bool valid = row < Nq;
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = valid ? qh[(size_t)row * D + c] : 0.f;
        acc[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    // Last key any row of this work-group attends.
    const int last_row = min(blockIdx.x * kRows + kRows, Nq) - 1;
    const int key_end = causal ? min(Nk, last_row + off + 1) : Nk;
    const int my_end = causal ? min(Nk, row + off + 1) : Nk;

    for (int t0 = 0; t0 < key_end; t0 += kTile) {
        // cooperative tile load (float4, coalesced); keys past Nk read as zero
        for (int e = tid; e < kTile * D / 4; e += kRows) {
            const int r = e / (D / 4), c4 = e % (D / 4);
            float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
            if (t0 + r < Nk) {
                kv4 = reinterpret_cast<const float4*>(kh + (size_t)(t0 + r) * D)[c4];
                vv4 = reinterpret_cast<const float4*>(vh + (size_t)(t0 + r) * D)[c4];
            }
            reinterpret_cast<float4*>(&ks[r][0])[c4] = kv4;
            reinterpret_cast<float4*>(&vs[r][0])[c4] = vv4;
        }
        __syncthreads();

        const int n = min(kTile, my_end - t0);  // keys of this tile the row attends
        if (n > 0) {
            float s[kTile];
            float mt = -INFINITY;
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                float dot = 0.f;
#pragma unroll
                for (int c = 0; c < D; ++c) dot = fmaf(qr[c], ks[j][c], dot);
                s[j] = j < n ? dot * scale : -INFINITY;
                mt = fmaxf(mt, s[j]);
            }
            const float m_new = fmaxf(m, mt);
            const float alpha = expf(m - m_new);  // 0 on the first tile (m = -inf)
            float lt = 0.f;
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                s[j] = expf(s[j] - m_new);       // masked keys give exp(-inf) = 0
                lt += s[j];
            }
            l = l * alpha + lt;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                float a = acc[c] * alpha;
#pragma unroll
                for (int j = 0; j < kTile; ++j) a = fmaf(s[j], vs[j][c], a);
                acc[c] = a;
            }
            m = m_new;
        }
        __syncthreads();
    }

    if (valid) {
        const float inv = 1.f / l;
        float* orow = o + (((size_t)b * H + h) * (size_t)Nq + row) * D;
#pragma unroll
        for (int c = 0; c < D; c += 4)
            *reinterpret_cast<float4*>(orow + c) =
                make_float4(acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv);
        if (lse) lse[((size_t)b * H + h) * (size_t)Nq + row] = m + logf(l);
    }
}

}  // namespace

hipError_t launch_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           hipStream_t stream) {
    dim3 grid((Nq + kRows - 1) / kRows, H, B);
    if (d == 64)
        hipLaunchKernelGGL(fwd_fp32_kernel<64>, grid, dim3(kRows), 0, stream, q, k, v, o, lse, H,
                           Hkv, Nq, Nk, causal, scale);
    else
        hipLaunchKernelGGL(fwd_fp32_kernel<128>, grid, dim3(kRows), 0, stream, q, k, v, o, lse,
                           H, Hkv, Nq, Nk, causal, scale);
    return hipGetLastError();
}

}  // namespace kvfa
