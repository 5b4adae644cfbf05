// rms_norm_bf16: RMSNorm with bf16 weights over a batch of tokens, gfx950.
//
// What it computes is the RMSNorm of the moeflux 0.1.0-pre.3 page
// src/riir/backend/gpu/gpu_norm.rs (documentation of `gpu_rms_norm_fused` and
// of the batched `encode_rms_norm_bf16_fused_n_tokens`): for every token t,
//     out[t,i] = x[t,i] * (1 / sqrt(sum_i x[t,i]^2 / dim + eps)) * w[i],
// with w the bf16 weight widened exactly.  As on the page, one workgroup of
// threads takes one token and the sum of squares never leaves the chip;
// unlike the page's two-dispatch single-token chain, the row is read once:
// when it fits (dim a multiple of 4, at most 8192) each thread keeps its
// 16-byte pieces of the row in registers between the reduction and the
// scaling, so the kernel moves x in and out once and is bound by HBM.  Rows
// of up to 2048 take one wave each (a reduction with no barrier).
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int kNormThreads = 256;

// Sum over the workgroup of NT threads; every thread receives the same bits
// (butterflies inside each wave, then the per-wave sums added in wave order).
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if constexpr (NT == 64) {
        return v;
    } else {
        const int wave = static_cast<int>(threadIdx.x) >> 6;
        if ((threadIdx.x & 63u) == 0) red[wave] = v;
        __syncthreads();
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) s += red[w];
        return s;
    }
}

__device__ __forceinline__ float rms_scale(float ss, uint32_t dim, float eps) {
    return 1.f / sqrtf(ss / static_cast<float>(dim) + eps);
}

// dim a multiple of 4, x and out 16-byte aligned, weight 8-byte aligned:
// thread j of NT holds the 16-byte pieces j, j + NT, ... (up to MAXV) of the
// row, so the row is read from HBM once and written once.
template <int NT, int MAXV>
__global__ __launch_bounds__(NT) void rms_norm_vec_kernel(
    const float* x, const uint16_t* __restrict__ w, float* out, uint32_t n_tokens, uint32_t dim,
    float eps)
{
    __shared__ float red[NT / 64];
    const uint32_t nv = dim / 4;
    for (uint32_t t = blockIdx.x; t < n_tokens; t += gridDim.x) {
        const size_t row = static_cast<size_t>(t) * dim;
        f32x4 v[MAXV];
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < MAXV; ++j) {
            const uint32_t p = threadIdx.x + j * NT;
            v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p < nv) v[j] = stream_load(reinterpret_cast<const f32x4*>(x + row) + p);
        }
#pragma unroll
        for (int j = 0; j < MAXV; ++j)
            ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
        const float r = rms_scale(block_sum<NT>(ss, red), dim, eps);
#pragma unroll
        for (int j = 0; j < MAXV; ++j) {
            const uint32_t p = threadIdx.x + j * NT;
            if (p < nv) {
                const u32x2 wb = *reinterpret_cast<const u32x2*>(w + 4 * p);
                const f32x4 o = {v[j].x * r * bf16_bits_to_f32(wb.x & 0xffffu),
                                 v[j].y * r * bf16_bits_to_f32(wb.x >> 16),
                                 v[j].z * r * bf16_bits_to_f32(wb.y & 0xffffu),
                                 v[j].w * r * bf16_bits_to_f32(wb.y >> 16)};
                stream_store(o, reinterpret_cast<f32x4*>(out + row) + p);
            }
        }
        if constexpr (NT > 64) __syncthreads();               // red is reused by the next token
    }
}

// Any dim and alignment: element by element, the row read twice (the second
// read comes from the cache hierarchy).  Every x element of a thread is read
// before any of them is written, and no thread writes an element another one
// reads, so out may be x itself.
__global__ __launch_bounds__(kNormThreads) void rms_norm_any_kernel(
    const float* x, const uint16_t* __restrict__ w, float* out, uint32_t n_tokens, uint32_t dim,
    float eps)
{
    __shared__ float red[kNormThreads / 64];
    for (uint32_t t = blockIdx.x; t < n_tokens; t += gridDim.x) {
        const size_t row = static_cast<size_t>(t) * dim;
        float ss = 0.f;
        for (uint32_t i = threadIdx.x; i < dim; i += kNormThreads) ss += x[row + i] * x[row + i];
        const float r = rms_scale(block_sum<kNormThreads>(ss, red), dim, eps);
        for (uint32_t i = threadIdx.x; i < dim; i += kNormThreads)
            out[row + i] = x[row + i] * r * bf16_bits_to_f32(w[i]);
        __syncthreads();                                      // red is reused by the next token
    }
}

}  // namespace

// One workgroup per token, up to this many workgroups; beyond, each one
// takes every kMaxNormGroups-th token (a launch covers at most 2^32 - 1
// work-items).
constexpr uint32_t kMaxNormGroups = 1u << 16;

template <int NT, int MAXV>
hipError_t launch_vec(const RmsNormArgs& a, hipStream_t stream) {
    const uint32_t grid = a.n_tokens < kMaxNormGroups ? a.n_tokens : kMaxNormGroups;
    hipLaunchKernelGGL((rms_norm_vec_kernel<NT, MAXV>), dim3(grid), dim3(NT), 0, stream,
                       a.x, a.weight, a.out, a.n_tokens, a.dim, a.eps);
    return hipGetLastError();
}

hipError_t launch_rms_norm(const RmsNormArgs& a, hipStream_t stream) {
    const bool vec = a.dim % 4 == 0 && reinterpret_cast<uintptr_t>(a.x) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(a.out) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(a.weight) % 8 == 0;
    const uint32_t nv = a.dim / 4;
    // One wave per token while a lane holds at most eight 16-byte pieces
    // (dim <= 2048): no barrier, and 8 KiB of the row in flight per wave.
    // Wider rows spread over 128 or 256 threads.
    if (vec && nv <= 64u * 8) {
        if (nv <= 64u * 2) return launch_vec<64, 2>(a, stream);
        if (nv <= 64u * 4) return launch_vec<64, 4>(a, stream);
        return launch_vec<64, 8>(a, stream);
    }
    if (vec && nv <= 128u * 8) return launch_vec<128, 8>(a, stream);
    if (vec && nv <= 256u * 8) return launch_vec<256, 8>(a, stream);
    const uint32_t grid = a.n_tokens < kMaxNormGroups ? a.n_tokens : kMaxNormGroups;
    hipLaunchKernelGGL(rms_norm_any_kernel, dim3(grid), dim3(kNormThreads), 0, stream, a.x,
                       a.weight, a.out, a.n_tokens, a.dim, a.eps);
    return hipGetLastError();
}

}  // namespace gdn
