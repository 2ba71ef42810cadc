// Reference kernels: the read stream, the MFMA-only and MFMA + epilogue loops behind
// the measured ceilings, and the two fp8 x e2m1 dot-product forms the fp8-query route
// chose between.

#include "idx_device.h"

namespace idx {
namespace {

// ---------------------------------------------------------------- measurement --
//
// Reference rates for the roofline, run on the same chip as the indexer: a plain
// read stream (what the K gather can at best reach) and an MFMA-only loop on the
// MX-FP4 instruction the scoring uses (what the contraction can at best reach).

constexpr int kMeasureThreads = 256;

// Every 16-byte word of src[0, n16) read once: thread g reads words g + j*T (T = all
// threads), eight non-temporal loads in flight (the fastest of the shapes measured:
// 6.3-6.5 TB/s), contiguous across the wave; an XOR of everything read goes to
// sink[workgroup] so the loads are live.
__global__ __launch_bounds__(kMeasureThreads) void measure_read_kernel(const uint4 *src, int64_t n16,
                                                                       uint32_t *sink) {
    const int64_t nthr = (int64_t)gridDim.x * kMeasureThreads;
    int64_t i = (int64_t)blockIdx.x * kMeasureThreads + threadIdx.x;
    uint32_t acc = 0;
    const v4u *s4 = reinterpret_cast<const v4u *>(src);
    for (; i + 7 * nthr < n16; i += 8 * nthr) {
        v4u v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(s4 + i + j * nthr);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    for (; i < n16; i += nthr) {
        const v4u a = __builtin_nontemporal_load(s4 + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
    __shared__ uint32_t w[kMeasureThreads / kWave];
    if ((threadIdx.x & (kWave - 1)) == 0) w[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int j = 0; j < kMeasureThreads / kWave; ++j) x ^= w[j];
        sink[blockIdx.x] = x;
    }
}

// The two ways of forming e4m3 x (e2m1 with UE8M0 block scales) dot products over 128
// dimensions, for 16 query rows against 16 tokens, one wave: (mode 0) the MX-scaled
// v_mfma_scale_f32_16x16x128_f8f6f4 on the raw codes (query scale bytes 127), and (mode 1)
// the fp8-query kernels' route: both operands converted exactly to bf16 (the token's
// scale applied in the conversion) and v_mfma_f32_16x16x32_bf16.  q: e4m3 [16][128];
// kv: packed e2m1 [16][64]; ks: UE8M0 [16][4]; out: fp32 [16 rows][16 tokens].
__global__ __launch_bounds__(kWave) void measure_fp8_dot_kernel(const uint8_t *q,
                                                                const uint8_t *kv,
                                                                const uint8_t *ks, int32_t mode,
                                                                float *out) {
    const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
    // B: token n, dimensions [32g, 32g + 32) as 16 bytes, and their scale byte
    const uint4 kb = *(const uint4 *)(kv + n * 64 + 16 * g);
    const int ksc = ks[n * 4 + g];
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (mode == 0 || mode == 2) {
        // A: row n, bytes j < 16 -> dimension 16g + j, bytes j >= 16 -> 64 + 16g + j - 16
        const uint4 a0 = *(const uint4 *)(q + n * 128 + 16 * g);
        const uint4 a1 = *(const uint4 *)(q + n * 128 + 64 + 16 * g);
        const v8i a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                          (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        if (mode == 0) {
            const v8i b = v8i{(int)kb.x, (int)kb.y, (int)kb.z, (int)kb.w, 0, 0, 0, 0};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 4, 0, 127, 0,
                                                                   ksc);
        } else {
            // B as e4m3 in A's layout: token n's e2m1 values of dimensions [16g, 16g+16)
            // (packed bytes [8g, 8g+8)) and [64+16g, 64+16g+16) (bytes [32+8g, 32+8g+8)),
            // each converted exactly (every e2m1 value is an e4m3 value)
            const uint2 k0 = *(const uint2 *)(kv + n * 64 + 8 * g);
            const uint2 k1 = *(const uint2 *)(kv + n * 64 + 32 + 8 * g);
            const uint32_t src[4] = {k0.x, k0.y, k1.x, k1.y};
            int b8[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t lo = 0u, hi = 0u;   // nibbles 0-3 and 4-7 of src[w], low first
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t c = (src[w] >> (4 * j)) & 15u, m = c & 7u;
                    const uint32_t e = (m == 0u ? 0u : m == 1u ? 0x30u : 0x38u + 4u * (m - 2u)) |
                                       ((c & 8u) << 4);
                    if (j < 4) lo |= e << (8 * j);
                    else hi |= e << (8 * (j - 4));
                }
                b8[2 * w] = (int)lo;
                b8[2 * w + 1] = (int)hi;
            }
            const v8i b = v8i{b8[0], b8[1], b8[2], b8[3], b8[4], b8[5], b8[6], b8[7]};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0,
                                                                   ksc);
        }
    } else {
        // A: row n, dimensions [32g, 32g + 32) as bf16 (the bf16 MFMA's k slot of step s,
        // lane group g, element j carries dimension 32g + 8s + j, as in load_q)
        const uint8_t *pq = q + n * 128 + 32 * g;
        const uint4 x = *(const uint4 *)pq, y = *(const uint4 *)(pq + 16);
        const uint32_t dq[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
        v8bf qa[4];
#pragma unroll
        for (int st = 0; st < 4; ++st)
            qa[st] = cat4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dq[2 * st], 1.0f, false),
                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dq[2 * st], 1.0f, true),
                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dq[2 * st + 1], 1.0f, false),
                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dq[2 * st + 1], 1.0f, true));
        KTile kt{kb, ksc};
        const float scale = __uint_as_float(ksc == 0 ? 0x00400000u
                                            : ksc == 0xFF ? 0x7FC00000u : (uint32_t)ksc << 23);
        const uint32_t d[4] = {kt.v.x, kt.v.y, kt.v.z, kt.v.w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const v8bf b = cat4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 0),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 1),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 2),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 3));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st], b, acc, 0, 0, 0);
        }
    }
    // C: lane holds token n, rows 4g + v
#pragma unroll
    for (int v = 0; v < 4; ++v) out[(4 * g + v) * 16 + n] = acc[v];
}

// Each wave: iters rounds of 8 independent v_mfma_scale_f32_16x16x128_f8f6f4 chains on
// e2m1 operands held in registers (nonzero codes that differ by lane; scale bytes
// 127), no memory traffic until one float per wave goes to sink.
__global__ __launch_bounds__(kMeasureThreads) void measure_mfma_kernel(int32_t iters, float *sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const int x = 0x3A5C1E72 ^ (lane * 0x01030507) ^ iters;
    const v8i a = v8i{x | 0x11111111, (x >> 3) | 0x22222222, (x << 5) | 0x11111111,
                      x ^ 0x7F3E1D2C, 0, 0, 0, 0};
    const v8i b = v8i{(x * 7) | 0x11111111, x ^ 0x5A5A5A5A, (x >> 7) | 0x33333333,
                      (x * 13) | 0x21212121, 0, 0, 0, 0};
    v4f acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 4, 4, 0, 127, 0,
                                                                      127);
    }
    float t = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) t += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    if (lane == 0) sink[blockIdx.x * (kMeasureThreads / kWave) + threadIdx.x / kWave] = t;
}

// The MFMA rate that the scoring epilogue leaves: the same 8 MX-FP4 MFMAs a round as
// measure_mfma_kernel, each a fresh product (C = 0, the B operand bumped by one VALU add),
// and every product's 4 accumulators folded through the ReLU-weight epilogue (an integer
// max and an fp32 FMA each), 9 VALU operations per MFMA, as the prefill scoring loop
// issues them.  Registers only; one float per wave goes to sink.
__global__ __launch_bounds__(kMeasureThreads) void measure_mfma_relu_kernel(int32_t iters,
                                                                           float *sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const int x = 0x3A5C1E72 ^ (lane * 0x01030507) ^ iters;
    const v8i a = v8i{x | 0x11111111, (x >> 3) | 0x22222222, (x << 5) | 0x11111111,
                      x ^ 0x7F3E1D2C, 0, 0, 0, 0};
    v8i b = v8i{(x * 7) | 0x11111111, x ^ 0x5A5A5A5A, (x >> 7) | 0x33333333,
                (x * 13) | 0x21212121, 0, 0, 0, 0};
    const float w[4] = {0.125f + lane * 1e-3f, 0.25f, -0.5f, 0.375f};
    float p = 0.0f;
    for (int it = 0; it < iters; ++it) {
        v4f r[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            b[0] += 0x10;
            r[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a, b, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0, 127, 0, 127);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) p = relu_weighted(w, r[c], p);
    }
    if (lane == 0) sink[blockIdx.x * (kMeasureThreads / kWave) + threadIdx.x / kWave] = p;
}

}  // namespace

hipError_t launch_measure_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
    hipLaunchKernelGGL(measure_read_kernel, dim3(kMeasureWgs), dim3(kMeasureThreads), 0, stream,
                       (const uint4 *)src, (int64_t)(bytes / 16), sink);
    return hipGetLastError();
}

hipError_t launch_measure_fp8_dot(const uint8_t *q, const uint8_t *kv, const uint8_t *ks,
                                  int32_t mode, float *out, hipStream_t stream) {
    hipLaunchKernelGGL(measure_fp8_dot_kernel, dim3(1), dim3(kWave), 0, stream, q, kv, ks, mode,
                       out);
    return hipGetLastError();
}

hipError_t launch_measure_mfma(int32_t iters, float *sink, hipStream_t stream) {
    hipLaunchKernelGGL(measure_mfma_kernel, dim3(kMeasureWgs), dim3(kMeasureThreads), 0, stream, iters,
                       sink);
    return hipGetLastError();
}

hipError_t launch_measure_mfma_relu(int32_t iters, float *sink, hipStream_t stream) {
    hipLaunchKernelGGL(measure_mfma_relu_kernel, dim3(kMeasureWgs), dim3(kMeasureThreads), 0, stream,
                       iters, sink);
    return hipGetLastError();
}

}  // namespace idx
