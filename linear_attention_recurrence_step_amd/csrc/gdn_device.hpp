// Device-side helpers shared by the gfx950 kernels of libgdn: I/O dtype
// conversion, vector memory access, 16-lane DPP reductions and the
// XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// I/O dtype codes (same values as gdn_dtype in include/gdn.h).
enum IoType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

template <int IO> struct IoTraits;
template <> struct IoTraits<kF32>  { static constexpr int kBytes = 4; };
template <> struct IoTraits<kF16>  { static constexpr int kBytes = 2; };
template <> struct IoTraits<kBF16> { static constexpr int kBytes = 2; };

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// Round to nearest, ties to even; any NaN becomes the canonical quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Hardware conversion (v_cvt_f16_f32) rounds to nearest even in the default mode.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <int IO>
__device__ __forceinline__ float io_load1(const void* base, size_t idx) {
    if constexpr (IO == kF32) {
        return static_cast<const float*>(base)[idx];
    } else if constexpr (IO == kBF16) {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
    } else {
        return f16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
    }
}

// ---------------------------------------------------------------- vectors

template <int BYTES> struct RawVec;
template <> struct RawVec<2>  { using T = uint16_t; };
template <> struct RawVec<4>  { using T = uint32_t; };
template <> struct RawVec<8>  { using T = uint2; };
template <> struct RawVec<16> { using T = uint4; };

// Load N consecutive I/O elements starting at element `idx` and widen them to
// float.  The address must be aligned to min(16, N * element size) bytes.
template <int IO, int N>
__device__ __forceinline__ void io_load_vec(const void* base, size_t idx, float (&out)[N]) {
    constexpr int EB = IoTraits<IO>::kBytes;
    constexpr int BYTES = N * EB;
    constexpr int PIECE = BYTES < 16 ? BYTES : 16;
    constexpr int NP = BYTES / PIECE;
    constexpr int PER = PIECE / EB;
    const char* p = static_cast<const char*>(base) + idx * EB;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        typename RawVec<PIECE>::T raw = *reinterpret_cast<const typename RawVec<PIECE>::T*>(p + i * PIECE);
        uint32_t w[PIECE / 4 > 0 ? PIECE / 4 : 1];
        if constexpr (PIECE >= 4) {
            __builtin_memcpy(w, &raw, PIECE);
        } else {
            w[0] = raw;
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            float f;
            if constexpr (IO == kF32) {
                f = __uint_as_float(w[e]);
            } else {
                uint32_t bits = (PIECE >= 4) ? ((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu) : w[0];
                f = (IO == kBF16) ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
            }
            out[i * PER + e] = f;
        }
    }
}

// Round N floats to the I/O dtype and store them at element `idx`.
template <int IO, int N>
__device__ __forceinline__ void io_store_vec(void* base, size_t idx, const float (&in)[N]) {
    constexpr int EB = IoTraits<IO>::kBytes;
    constexpr int BYTES = N * EB;
    constexpr int PIECE = BYTES < 16 ? BYTES : 16;
    constexpr int NP = BYTES / PIECE;
    constexpr int PER = PIECE / EB;
    char* p = static_cast<char*>(base) + idx * EB;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        typename RawVec<PIECE>::T raw;
        if constexpr (IO == kF32) {
            uint32_t w[PER];
#pragma unroll
            for (int e = 0; e < PER; ++e) w[e] = __float_as_uint(in[i * PER + e]);
            __builtin_memcpy(&raw, w, PIECE);
        } else if constexpr (PIECE >= 4) {
            uint32_t w[PIECE / 4];
#pragma unroll
            for (int e = 0; e < PIECE / 4; ++e) {
                float a = in[i * PER + 2 * e], b = in[i * PER + 2 * e + 1];
                uint32_t lo = (IO == kBF16) ? f32_to_bf16_bits(a) : f32_to_f16_bits(a);
                uint32_t hi = (IO == kBF16) ? f32_to_bf16_bits(b) : f32_to_f16_bits(b);
                w[e] = lo | (hi << 16);
            }
            __builtin_memcpy(&raw, w, PIECE);
        } else {
            float a = in[i * PER];
            raw = static_cast<uint16_t>((IO == kBF16) ? f32_to_bf16_bits(a) : f32_to_f16_bits(a));
        }
        *reinterpret_cast<typename RawVec<PIECE>::T*>(p + i * PIECE) = raw;
    }
}

// N consecutive float32 values (the recurrent state); 8- or 16-byte aligned.
template <int N>
__device__ __forceinline__ void f32_load_vec(const float* p, float (&out)[N]) {
    static_assert(N == 2 || N == 4, "state chunks are 2 or 4 floats");
    if constexpr (N == 4) {
        float4 v = *reinterpret_cast<const float4*>(p);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    } else {
        float2 v = *reinterpret_cast<const float2*>(p);
        out[0] = v.x; out[1] = v.y;
    }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Non-temporal store of N floats: the state written back is not re-read by
// this launch, so it should not displace reusable lines from the caches.
template <int N>
__device__ __forceinline__ void f32_store_vec_nt(float* p, const float (&in)[N]) {
    static_assert(N == 2 || N == 4, "state chunks are 2 or 4 floats");
    if constexpr (N == 4) {
        f32x4 v = {in[0], in[1], in[2], in[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
    } else {
        f32x2 v = {in[0], in[1]};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x2*>(p));
    }
}

// ------------------------------------------------------------ reductions

template <int CTRL>
__device__ __forceinline__ float dpp_read(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the same
// bits (each butterfly stage adds the same two partial sums on both sides).
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_read<0xb1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_read<0x4e>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp_read<0x141>(x);  // row_half_mirror: quads 0<->1, 2<->3
    x += dpp_read<0x140>(x);  // row_mirror: half-rows swap
    return x;
}

// ------------------------------------------------- workgroup ordering

// Workgroups are handed to the 8 XCDs round-robin (block i -> XCD i % 8).
// Renumber them so that each XCD receives one contiguous range of logical
// indices: neighbouring logical work (the row blocks of one head, the value
// heads sharing a key head) then shares that XCD's L2.
__device__ __forceinline__ uint32_t xcd_contiguous_index(uint32_t bid, uint32_t nblk) {
    constexpr uint32_t kXcd = 8;
    const uint32_t xcd = bid % kXcd;
    const uint32_t idx = bid / kXcd;
    const uint32_t per = nblk / kXcd;
    const uint32_t rem = nblk % kXcd;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

}  // namespace gdn
