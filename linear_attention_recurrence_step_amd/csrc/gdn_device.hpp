// Device-side helpers shared by the gfx950 kernels of libgdn: I/O dtype
// conversion, vector memory access, 16-lane DPP reductions and the
// XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

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

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int BYTES> struct RawVec;
template <> struct RawVec<2>  { using T = uint16_t; };
template <> struct RawVec<4>  { using T = uint32_t; };
template <> struct RawVec<8>  { using T = u32x2; };
template <> struct RawVec<16> { using T = u32x4; };

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

// Bit copy of N consecutive I/O elements (aligned to min(16, N * element size)).
template <int IO, int N>
__device__ __forceinline__ void io_copy_vec(const void* src, size_t si, void* dst, size_t di) {
    constexpr int EB = IoTraits<IO>::kBytes;
    constexpr int BYTES = N * EB;
    constexpr int PIECE = BYTES < 16 ? BYTES : 16;
    using V = typename RawVec<PIECE>::T;
    const char* s = static_cast<const char*>(src) + si * EB;
    char* d = static_cast<char*>(dst) + di * EB;
#pragma unroll
    for (int i = 0; i < BYTES / PIECE; ++i)
        *reinterpret_cast<V*>(d + i * PIECE) = *reinterpret_cast<const V*>(s + i * PIECE);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// N consecutive I/O elements held as their raw bits (in pieces of at most 16
// bytes), widened only where they are used, so that a load is never waited
// for where it is issued.
template <int IO, int N>
struct RawIo {
    static constexpr int EB = IoTraits<IO>::kBytes;
    static constexpr int BYTES = N * EB;
    static constexpr int PB = BYTES < 16 ? BYTES : 16;       // bytes per piece
    static constexpr int NP = BYTES / PB;
    static constexpr int PER = PB / EB;                      // elements per piece
    using V = typename RawVec<PB>::T;
    V raw[NP];
    __device__ __forceinline__ void load(const void* base, size_t idx) {
        const char* p = static_cast<const char*>(base) + idx * EB;
#pragma unroll
        for (int i = 0; i < NP; ++i) raw[i] = *reinterpret_cast<const V*>(p + i * PB);
    }
    __device__ __forceinline__ void store(void* base, size_t idx) const {
        char* p = static_cast<char*>(base) + idx * EB;
#pragma unroll
        for (int i = 0; i < NP; ++i) *reinterpret_cast<V*>(p + i * PB) = raw[i];
    }
    __device__ __forceinline__ float at(int e) const {
        const V& piece = raw[e / PER];
        const int j = e % PER;
        if constexpr (PB >= 4) {
            uint32_t w[PB / 4];
            __builtin_memcpy(w, &piece, PB);
            if constexpr (IO == kF32) return __uint_as_float(w[j]);
            const uint32_t bits = (w[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
            return IO == kBF16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
        } else {
            const uint32_t bits = piece;
            return IO == kBF16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
        }
    }
};


// Streaming accesses: data that one launch reads once (the recurrent state,
// a tape, a source to copy) or writes once, with the non-temporal hint both
// ways.  Non-temporal stores measured faster than plain ones where it counts:
// back-to-back decode steps over inputs too large to stay in the caches
// (every write-back paid inside the timing) ran 355 us a step with them and
// 372 us with plain stores (380 us with plain loads too).  Timed in
// isolation after a cache scrub, plain stores look faster, because up to a
// cache's worth of their write-backs is left for whatever runs next.
template <typename V>
__device__ __forceinline__ V stream_load(const V* p) {
    return __builtin_nontemporal_load(p);
}
template <typename V>
__device__ __forceinline__ void stream_store(V v, V* p) {
    __builtin_nontemporal_store(v, p);
}

// N consecutive float32 values of the state (read once per launch); 8- or
// 16-byte aligned.
template <int N>
__device__ __forceinline__ void f32_load_vec(const float* p, float (&out)[N]) {
    static_assert(N == 2 || N == 4, "state chunks are 2 or 4 floats");
    if constexpr (N == 4) {
        f32x4 v = stream_load(reinterpret_cast<const f32x4*>(p));
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    } else {
        f32x2 v = stream_load(reinterpret_cast<const f32x2*>(p));
        out[0] = v.x; out[1] = v.y;
    }
}

// N floats of the state, written once per launch.
template <int N>
__device__ __forceinline__ void f32_store_vec(float* p, const float (&in)[N]) {
    static_assert(N == 2 || N == 4, "state chunks are 2 or 4 floats");
    if constexpr (N == 4) {
        stream_store(f32x4{in[0], in[1], in[2], in[3]}, reinterpret_cast<f32x4*>(p));
    } else {
        stream_store(f32x2{in[0], in[1]}, reinterpret_cast<f32x2*>(p));
    }
}

// A thread's RPT consecutive state rows (row r at p + r * 16 * E floats),
// lane `lane` holding the columns {(c * 16 + lane) * W + w} of each.  The
// rows are visited by a fold, not a loop: a one-trip loop over the rows (one
// row per thread) survived until the backend's loop-invariant code motion,
// which rewrote its stores without the non-temporal hint.
template <int E, size_t... R>
__device__ __forceinline__ void load_rows_impl(const float* p, uint32_t lane, float (&s)[sizeof...(R)][E],
                                               std::index_sequence<R...>) {
    constexpr int W = E < 4 ? E : 4;
    auto one = [&](const float* row, float (&dst)[E]) {
#pragma unroll
        for (int c = 0; c < E / W; ++c) {
            float t[W];
            f32_load_vec<W>(row + (c * 16 + lane) * W, t);
#pragma unroll
            for (int w = 0; w < W; ++w) dst[c * W + w] = t[w];
        }
    };
    (one(p + R * 16 * E, s[R]), ...);
}
template <int E, size_t... R>
__device__ __forceinline__ void store_rows_impl(float* p, uint32_t lane, const float (&s)[sizeof...(R)][E],
                                                std::index_sequence<R...>) {
    constexpr int W = E < 4 ? E : 4;
    auto one = [&](float* row, const float (&src)[E]) {
#pragma unroll
        for (int c = 0; c < E / W; ++c) {
            float t[W];
#pragma unroll
            for (int w = 0; w < W; ++w) t[w] = src[c * W + w];
            f32_store_vec<W>(row + (c * 16 + lane) * W, t);
        }
    };
    (one(p + R * 16 * E, s[R]), ...);
}
template <int RPT, int E>
__device__ __forceinline__ void load_state_rows(const float* p, uint32_t lane, float (&s)[RPT][E]) {
    load_rows_impl<E>(p, lane, s, std::make_index_sequence<RPT>{});
}
template <int RPT, int E>
__device__ __forceinline__ void store_state_rows(float* p, uint32_t lane, const float (&s)[RPT][E]) {
    store_rows_impl<E>(p, lane, s, std::make_index_sequence<RPT>{});
}

// Wait until every vector memory load and store issued so far has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left unconstrained).  Issued once
// after a kernel's initial state loads: otherwise the compiler treats those
// registers as possibly still loading inside later loops and waits on the
// in-order counter there, which also waits for any prefetch issued meanwhile.
__device__ __forceinline__ void wait_vector_memory() {
    __builtin_amdgcn_s_waitcnt(0x0f70);
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

// Row sums of N independent values at once: the stages are interleaved so
// the wait states a DPP read needs after a VALU write are filled with the
// other values' work.  Same bits as N separate row16_sum calls.
template <int N>
__device__ __forceinline__ void row16_sum_n(float (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_read<0xb1>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_read<0x4e>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_read<0x141>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_read<0x140>(x[i]);
}

// ------------------------------------------------- workgroup ordering

// Workgroups are handed to the 8 XCDs round-robin (block i -> XCD i % 8).
// Renumber them so that each XCD receives one contiguous range of logical
// indices: neighbouring logical work (the row blocks of one head, and under
// the block map the value heads sharing a key head) then shares that XCD's L2.
__device__ __forceinline__ uint32_t xcd_contiguous_index(uint32_t bid, uint32_t nblk) {
    constexpr uint32_t kXcd = 8;
    const uint32_t xcd = bid % kXcd;
    const uint32_t idx = bid / kXcd;
    const uint32_t per = nblk / kXcd;
    const uint32_t rem = nblk % kXcd;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

}  // namespace gdn

namespace gdn {

// ------------------------------------------------------- chunk staging

// LDS vector access of N floats; the address must be aligned to
// min(16, 4 * N) bytes (N = 1, 2, 4 or a multiple of 4).
template <int N>
__device__ __forceinline__ void lds_store_vec(float* p, const float (&f)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4)
            *reinterpret_cast<f32x4*>(p + i) = f32x4{f[i], f[i + 1], f[i + 2], f[i + 3]};
    } else if constexpr (N == 2) {
        *reinterpret_cast<f32x2*>(p) = f32x2{f[0], f[1]};
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) p[i] = f[i];
    }
}

template <int N>
__device__ __forceinline__ void lds_load_vec(const float* p, float (&f)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
            f[i] = v.x; f[i + 1] = v.y; f[i + 2] = v.z; f[i + 3] = v.w;
        }
    } else if constexpr (N == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(p);
        f[0] = v.x; f[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) f[i] = p[i];
    }
}

// Cooperative copy of a [ROWS x COLS] block of I/O elements into LDS as
// float32, split into a global-load phase (into registers) and an LDS-store
// phase, so the loads of the next chunk of steps can be in flight while the
// current chunk is being computed.  Source row i starts `stride` elements
// after row i-1; pieces of P contiguous elements (P * element size <= 16
// bytes, P dividing COLS) are spread over the NT threads of the workgroup.
// Rows i >= valid (past the end of the tape) are not loaded and hold zeros.
// Rows of inactive steps are loaded like any other (their consumers skip
// them); predicating each load on its mask entry would put a dependent load
// in front of every piece.
template <int IO, int ROWS, int COLS, int P, int NT>
struct ChunkStager {
    static constexpr int EB = IoTraits<IO>::kBytes;
    static constexpr int PER_ROW = COLS / P;
    static constexpr int PIECES = ROWS * PER_ROW;
    static constexpr int PER_THREAD = (PIECES + NT - 1) / NT;
    using Raw = typename RawVec<P * EB>::T;
    static_assert(COLS % P == 0 && P * EB <= 16, "bad piece size");

    Raw buf[PER_THREAD];

    __device__ __forceinline__ void load(const void* src, size_t stride, int valid) {
        const char* base = static_cast<const char*>(src);
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int p = static_cast<int>(threadIdx.x) + j * NT;
            buf[j] = Raw{};
            if (p < PIECES) {
                const int row = p / PER_ROW;
                const int col = (p - row * PER_ROW) * P;
                if (row < valid)
                    buf[j] = *reinterpret_cast<const Raw*>(base + (static_cast<size_t>(row) * stride + col) * EB);
            }
        }
    }

    // Rows [0, rows) go to LDS (rows <= ROWS: the LDS block may be shorter
    // than the chunk when the whole tape is shorter).
    __device__ __forceinline__ void store(float* lds, int rows) const {
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int p = static_cast<int>(threadIdx.x) + j * NT;
            if (p < PIECES && p < rows * PER_ROW) {
                const int row = p / PER_ROW;
                const int col = (p - row * PER_ROW) * P;
                float f[P];
                unpack(buf[j], f);
                lds_store_vec<P>(lds + row * COLS + col, f);
            }
        }
    }

    // The raw (unconverted) pieces to global memory: row i of the block goes to
    // dst + i * stride elements, for rows i < valid whose step flag is set
    // (flags are read from LDS at flag4[4 * i]; NULL: every row).  A bit copy.
    __device__ __forceinline__ void store_global(void* dst, size_t stride, int valid,
                                                 const float* flag4) const {
        char* base = static_cast<char*>(dst);
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int p = static_cast<int>(threadIdx.x) + j * NT;
            if (p < PIECES) {
                const int row = p / PER_ROW;
                const int col = (p - row * PER_ROW) * P;
                if (row < valid && (flag4 == nullptr || __float_as_uint(flag4[4 * row]) != 0u))
                    *reinterpret_cast<Raw*>(base + (static_cast<size_t>(row) * stride + col) * EB) = buf[j];
            }
        }
    }

    // For single-column blocks: row i goes to lds[i * stride]; rows at or
    // past `valid` (not loaded) get `pad` instead.
    __device__ __forceinline__ void store_strided(float* lds, int stride, int rows, int valid,
                                                  float pad) const {
        static_assert(COLS == 1 && P == 1, "strided store is for one value per row");
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int p = static_cast<int>(threadIdx.x) + j * NT;
            if (p < PIECES && p < rows) {
                float f[1];
                unpack(buf[j], f);
                lds[p * stride] = p < valid ? f[0] : pad;
            }
        }
    }

  private:
    __device__ __forceinline__ static void unpack(const Raw& raw, float (&f)[P]) {
        if constexpr (P * EB >= 4) {
            uint32_t w[(P * EB) / 4];
            __builtin_memcpy(w, &raw, P * EB);
#pragma unroll
            for (int e = 0; e < P; ++e) {
                if constexpr (IO == kF32) {
                    f[e] = __uint_as_float(w[e]);
                } else {
                    const uint32_t bits = (w[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                    f[e] = (IO == kBF16) ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
                }
            }
        } else {
            const uint32_t bits = raw;
            f[0] = (IO == kBF16) ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
        }
    }
};

// Mask entries of a chunk of steps (1 when there is no mask), for LDS.
template <int ROWS, int NT>
struct MaskStager {
    static constexpr int PER_THREAD = (ROWS + NT - 1) / NT;
    uint32_t buf[PER_THREAD];
    __device__ __forceinline__ void load(const uint32_t* mask_row, int valid) {
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int p = static_cast<int>(threadIdx.x) + j * NT;
            buf[j] = 0u;
            if (p < ROWS && p < valid) buf[j] = mask_row == nullptr ? 1u : mask_row[p];
        }
    }
    __device__ __forceinline__ void store(uint32_t* lds, int rows) const { store_strided(lds, 1, rows); }
    __device__ __forceinline__ void store_strided(uint32_t* lds, int stride, int rows) const {
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int p = static_cast<int>(threadIdx.x) + j * NT;
            if (p < ROWS && p < rows) lds[p * stride] = buf[j];
        }
    }
};

// Widest piece (in elements) for a row of COLS I/O elements: at most 16 bytes.
template <int IO, int COLS>
constexpr int piece_elems() {
    constexpr int max_p = 16 / IoTraits<IO>::kBytes;
    int p = max_p;
    while (p > 1 && COLS % p != 0) p >>= 1;
    return p;
}

}  // namespace gdn
