// gdn_replay for long folds of a 16-bit tape: the fold as a matrix product on
// the matrix cores, gfx950.
//
// What it computes is the replay kernel (macro `state_replay!`) of the
// metaltile-std 0.1.0 page src/ffai/gated_delta_replay.rs, the same as
// gdn_replay.hip.  Unrolled over a chunk of C tape positions, the fold
// S <- g_t S + delta_t k_t^T (taken positions only) is
//     S <- gamma * S + sum_t w_t * delta_t k_t^T,
// with gamma the product of the chunk's taken gates and w_t the product of the
// taken gates after t within the chunk (w_t = 0 for an untaken t).  The sum is
// a [Dv x C] x [C x Dk] product contracted over positions: a dense contraction,
// which runs here on v_mfma_f32_16x16x16 with fp32 accumulation instead of one
// VALU FMA per state value per position.
//
// Operands.  The state is accumulated transposed, S^T [Dk x Dv], so each lane
// of a 16x16 accumulator tile holds four consecutive Dk columns of one state
// row and the state moves in 16-byte vectors.  A = k^T [Dk x C] enters exactly
// (the tape's own 16-bit values).  B = (w_t delta_t) [C x Dv] is fp32 and enters
// as the sum of two 16-bit numbers, hi = round(x) and lo = round(x - hi) (two
// MFMAs), keeping about 22 significant bits for fp16 tapes and 16 for bf16.
// With every taken gate of the chunk in [0, 1], |w_t| <= 1, so w_t delta_t
// stays within the tape dtype's range; a chunk with any other taken gate (or a
// NaN gate) runs the exact sequential update instead, one position per MFMA,
// on the state itself (see the fold below).
// Positions past `accepted` are never loaded.  Masked positions below it are
// loaded with the rest of their chunk (unconditional loads keep the
// compiler's memory waits exact) but their rows of A and B are zeroed before
// they reach an operand, so a NaN in an untaken slot cannot reach S.
//
// Mapping.  A workgroup of NW waves takes 16*NW consecutive value rows of one
// head; each wave owns 16 rows across all Dk/16 column tiles (4*Dk/16 fp32
// accumulators per lane).  A chunk of 32 positions of k_log and delta_log is
// staged through LDS transposed ([column][position pair]), so each MFMA
// operand fragment (four consecutive positions) is one 8-byte LDS read.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int kPos = 32;        // tape positions per chunk: two MFMA contraction steps of 16
constexpr int kPairs = kPos / 2;
constexpr int kStride = kPairs + 2;  // LDS row stride in position pairs (dwords); the pad spreads banks

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// acc += A (16 x 16, four consecutive positions per lane) * B (16 x 16).
template <int IO>
__device__ __forceinline__ f32x4v mfma16(u32x2 a, u32x2 b, f32x4v acc) {
    if constexpr (IO == kF16)
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                         __builtin_bit_cast(i16x4, b), acc, 0, 0, 0);
}

template <int IO>
__device__ __forceinline__ float half_to_f32(uint32_t bits) {
    return IO == kF16 ? f16_bits_to_f32(bits) : bf16_bits_to_f32(bits);
}

// Raw bits of one 16-bit element, widened later (so the load is not waited
// for where it is issued).
template <int IO>
__device__ __forceinline__ uint32_t io_load_bits(const void* base, size_t idx) {
    return *reinterpret_cast<const uint16_t*>(static_cast<const char*>(base) + idx * 2);
}

template <int IO>
__device__ __forceinline__ float io_bits_to_f32(uint32_t bits) {
    return IO == kF16 ? f16_bits_to_f32(bits) : bf16_bits_to_f32(bits);
}

template <int IO>
__device__ __forceinline__ uint32_t f32_to_half(float f) {
    return IO == kF16 ? f32_to_f16_bits(f) : f32_to_bf16_bits(f);
}

// Split x into hi + lo, both in the 16-bit dtype: hi = round(x), lo = round(x - hi).
template <int IO>
__device__ __forceinline__ void split2(float x, uint32_t& hi, uint32_t& lo) {
    hi = f32_to_half<IO>(x);
    lo = f32_to_half<IO>(x - half_to_f32<IO>(hi));
}

template <int DK, int NW>
struct MfmaLds {
    static constexpr int ROWS = 16 * NW;                          // value rows per workgroup
    static constexpr int SROW = DK * 4 + 16;                      // padded state row in LDS (bytes)
    static constexpr int STATE = NW * 16 * SROW;                  // state transposition area
    static constexpr int KT = DK * kStride * 4;                   // chunk of k, [column][pair]
    static constexpr int DT = ROWS * kStride * 4;                 // chunk of delta, [row][pair]
    static constexpr int CHUNK = KT + DT + 3 * kPos * 4 + 16;     // + weights, gates, flags, misc
    static constexpr int BYTES = STATE > CHUNK ? STATE : CHUNK;   // the two are never live together
};

template <int IO, int DK, int NW, bool MASKED>
__global__ __launch_bounds__(64 * NW, DK <= 128 ? 4 : 2) void gdn_replay_mfma_kernel(
    const void* __restrict__ delta_log, const void* __restrict__ k_log,
    const void* __restrict__ g_log, const float* state_in,
    const uint32_t* __restrict__ mask, float* state_out,
    uint32_t T_log, uint32_t Hv, uint32_t Dv, uint32_t slices, uint32_t steps)
{
    using Lds = MfmaLds<DK, NW>;
    constexpr int NT = 64 * NW;
    constexpr int ROWS = Lds::ROWS;
    constexpr int NI = DK / 16;                               // column tiles = 16-byte state pieces per lane
    constexpr int KG = DK / 8, DG = ROWS / 8;                 // 8-element groups of a k / delta row
    constexpr int KPT = (kPairs * KG + NT - 1) / NT;          // (position pair, group) jobs per thread
    constexpr int DPT = (kPairs * DG + NT - 1) / NT;
    const uint32_t tid = threadIdx.x;
    const uint32_t l = tid & 63u;
    const uint32_t wave = tid >> 6;
    const uint32_t lr = l & 15u, lg = l >> 4;                 // fragment row, group of 4

    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const uint32_t n = blk / slices;                          // b * Hv + hv
    const uint32_t dv0 = (blk - n * slices) * ROWS;
    const uint32_t b = n / Hv;
    const uint32_t hv = n - b * Hv;

    __shared__ __align__(16) unsigned char lds[Lds::BYTES];
    unsigned char* sbuf = lds + wave * 16 * Lds::SROW;         // this wave's 16 state rows
    uint32_t* kT = reinterpret_cast<uint32_t*>(lds);
    uint32_t* dT = reinterpret_cast<uint32_t*>(lds + Lds::KT);
    float* wv = reinterpret_cast<float*>(lds + Lds::KT + Lds::DT);
    float* gs = wv + kPos;
    uint32_t* fl = reinterpret_cast<uint32_t*>(gs + kPos);
    float* misc = reinterpret_cast<float*>(fl + kPos);        // gamma of the chunk, chunk-ok flag

    // The wave's 16 rows move between HBM and registers row-contiguously
    // (piece p = l + 64u is 16 bytes of row p / (DK/4)), and between that
    // layout and the MFMA accumulator layout through LDS.
    const float* sin = state_in + (static_cast<size_t>(n) * Dv + dv0 + wave * 16) * DK;
    float* sout = state_out + (static_cast<size_t>(n) * Dv + dv0 + wave * 16) * DK;
    auto piece_lds = [&](int u) {
        const int p = static_cast<int>(l) + 64 * u;
        return sbuf + (p / (DK / 4)) * Lds::SROW + (p % (DK / 4)) * 16;
    };
    auto frag_lds = [&](int i) { return sbuf + lr * Lds::SROW + (4 * i + lg) * 16; };

    // Registers of the chunk in flight: job u of this thread covers positions
    // 2q, 2q+1 and 8-element group cg, with q = job / groups and cg = job mod
    // groups, so each row is read contiguously.  Every slot below `steps` is
    // loaded; untaken ones are zeroed when written to LDS.
    u32x4 kr[KPT][2], dr[DPT][2];
    uint32_t kmw[KPT][2], dmw[DPT][2], gmw, graw;
    const char* kb = static_cast<const char*>(k_log);
    const char* db = static_cast<const char*>(delta_log);
    // Every load below is unconditional, from an index clamped into the chunk
    // (straight-line code keeps the compiler's wait counts exact, so waiting
    // for one chunk never waits for loads issued after it); what a clamped
    // load brought in is discarded when the chunk is written to LDS.
    auto mask_at = [&](uint32_t t) -> uint32_t {
        if constexpr (MASKED) return mask[static_cast<size_t>(b) * T_log + t];
        else return 1u;
    };
    auto load_chunk = [&](uint32_t t0) {
        const int last = static_cast<int>(steps - t0 < kPos ? steps - t0 : kPos) - 1;
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            int jb = static_cast<int>(tid) + u * NT;
            jb = jb < kPairs * KG ? jb : kPairs * KG - 1;
            const int q = jb / KG, cg = jb - q * KG;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tt = 2 * q + h < last ? 2 * q + h : last;
                const size_t bt = static_cast<size_t>(b) * T_log + t0 + tt;
                kr[u][h] = stream_load(
                    reinterpret_cast<const u32x4*>(kb + ((bt * Hv + hv) * DK + cg * 8) * 2));
                kmw[u][h] = mask_at(t0 + tt);
            }
        }
#pragma unroll
        for (int u = 0; u < DPT; ++u) {
            int jb = static_cast<int>(tid) + u * NT;
            jb = jb < kPairs * DG ? jb : kPairs * DG - 1;
            const int q = jb / DG, dg = jb - q * DG;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tt = 2 * q + h < last ? 2 * q + h : last;
                const size_t bt = static_cast<size_t>(b) * T_log + t0 + tt;
                dr[u][h] = stream_load(
                    reinterpret_cast<const u32x4*>(db + ((bt * Hv + hv) * Dv + dv0 + dg * 8) * 2));
                dmw[u][h] = mask_at(t0 + tt);
            }
        }
        {                                                     // gate and mask of position tid (wave 0)
            const int tt = static_cast<int>(l) < last ? static_cast<int>(l) : last;
            gmw = mask_at(t0 + tt);
            graw = io_load_bits<IO>(g_log, (static_cast<size_t>(b) * T_log + t0 + tt) * Hv + hv);
        }
    };
    // Positions 2q, 2q+1 of element e of two 8-element rows, packed in one dword.
    auto pair_word = [](const u32x4& r0, const u32x4& r1, int e) {
        const uint32_t a = (r0[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        const uint32_t c = (r1[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        return a | (c << 16);
    };

    // The fold is accumulated apart from the state, U = sum over chunks of
    // (later gammas) * (chunk's w-weighted products), starting from zero, and
    // S = Gamma * S0 + U at the end (Gamma = product of every taken gate).  So
    // the state loads (issued with a single chunk, or while the last chunk of
    // a longer fold is folded) are in flight during the fold, and they never
    // hold registers at the same time as a prefetched chunk.  acc[i] is the
    // 16x16 tile of U^T for columns 16i.. and the wave's 16 rows; lane l holds
    // columns 16i + 4*lg + 0..3 of row lr.
    //
    // Gamma and U apart are only safe while every taken gate lies in [0, 1]
    // (Gamma then stays in [0, 1]).  The first chunk with any other gate
    // first folds the snapshot in, acc = Gamma * S0 + U, read straight from
    // memory in the accumulator layout, and from then on the accumulators
    // hold the state itself (`absorbed`): a long run of gates above 1 grows
    // the state step by step as the sequential fold does, instead of
    // overflowing a separate Gamma, and an infinite gate meets the state,
    // not an accumulator of zeros.
    f32x4 sreg[NI];
    auto load_state = [&]() {
#pragma unroll
        for (int u = 0; u < NI; ++u)
            sreg[u] = stream_load(reinterpret_cast<const f32x4*>(sin + (l + 64 * u) * 4));
    };
    f32x4v acc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[i] = f32x4v{0.f, 0.f, 0.f, 0.f};
    float Gamma = 1.f;
    bool absorbed = false;                                    // acc holds S itself (uniform)

    auto chunk = [&](uint32_t t0, auto prefetch) {
        const int valid = static_cast<int>(steps - t0 < kPos ? steps - t0 : kPos);
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int jb = static_cast<int>(tid) + u * NT;
            if (jb < kPairs * KG) {
                const int q = jb / KG, cg = jb - q * KG;
                const u32x4 z = {0u, 0u, 0u, 0u};
                const u32x4 r0 = 2 * q < valid && kmw[u][0] != 0u ? kr[u][0] : z;
                const u32x4 r1 = 2 * q + 1 < valid && kmw[u][1] != 0u ? kr[u][1] : z;
#pragma unroll
                for (int e = 0; e < 8; ++e) kT[(cg * 8 + e) * kStride + q] = pair_word(r0, r1, e);
            }
        }
#pragma unroll
        for (int u = 0; u < DPT; ++u) {
            const int jb = static_cast<int>(tid) + u * NT;
            if (jb < kPairs * DG) {
                const int q = jb / DG, dg = jb - q * DG;
                const u32x4 z = {0u, 0u, 0u, 0u};
                const u32x4 r0 = 2 * q < valid && dmw[u][0] != 0u ? dr[u][0] : z;
                const u32x4 r1 = 2 * q + 1 < valid && dmw[u][1] != 0u ? dr[u][1] : z;
#pragma unroll
                for (int e = 0; e < 8; ++e) dT[(dg * 8 + e) * kStride + q] = pair_word(r0, r1, e);
            }
        }
        if (tid < 64) {
            // Wave 0: the chunk's gates and flags (lane t holds position t),
            // and w_t = product of the taken gates after t by a suffix scan;
            // gamma = product of all.
            const int t = static_cast<int>(tid);
            const bool mine = t < valid && gmw != 0u;
            const float gt = mine ? io_bits_to_f32<IO>(graw) : 1.f;
            float p = gt;                                     // becomes prod_{s >= t} f_s
#pragma unroll
            for (int d = 1; d < kPos; d *= 2) {
                const float y = __shfl_down(p, d, kPos);
                if (t + d < kPos) p *= y;
            }
            const float after = __shfl_down(p, 1, kPos);
            const bool bad = mine && !(gt >= 0.f && gt <= 1.f);
            const bool ok = __ballot(bad) == 0ull;
            if (t < kPos) {
                fl[t] = mine ? 1u : 0u;
                gs[t] = mine ? gt : 0.f;
                wv[t] = mine ? (t + 1 < kPos ? after : 1.f) : 0.f;
                if (t == 0) {
                    misc[0] = p;
                    misc[1] = ok ? 1.f : 0.f;
                }
            }
        }
        __syncthreads();
        prefetch();                                           // in flight during this chunk

        // One pass over the chunk when its gates allow (w and gamma from the
        // chunk), else one pass per taken position (gamma = that gate, w = 1,
        // every other position's operand lanes zeroed), which is the exact
        // sequential update: each product then rounds like fma(k, delta, S * g).
        const bool whole = misc[1] != 0.f;
        if (!whole && !absorbed) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const f32x4 s0 = *reinterpret_cast<const f32x4*>(sin + lr * DK + 16 * i + 4 * lg);
                acc[i] = f32x4v{fmaf(Gamma, s0.x, acc[i][0]), fmaf(Gamma, s0.y, acc[i][1]),
                                fmaf(Gamma, s0.z, acc[i][2]), fmaf(Gamma, s0.w, acc[i][3])};
            }
            Gamma = 1.f;
            absorbed = true;
        }
        int tt = 0;
        for (;;) {
            float gamma = misc[0];
            uint64_t keep[2] = {~0ull, ~0ull};
            int only = -1;                                    // the one contraction step used, if any
            if (!whole) {
                while (tt < valid && fl[tt] == 0u) ++tt;
                if (tt >= valid) break;
                gamma = gs[tt];
                const uint64_t m = (static_cast<uint32_t>(tt & 15) >> 2) == lg ? 0xffffull << ((tt & 3) * 16) : 0ull;
                only = tt >> 4;
                keep[0] = only == 0 ? m : 0ull;
                keep[1] = only == 1 ? m : 0ull;
                ++tt;
            }
            Gamma *= gamma;
#pragma unroll
            for (int i = 0; i < NI; ++i) acc[i] *= gamma;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (whole ? 16 * ks >= valid : only != ks) continue;
                float w4[4] = {1.f, 1.f, 1.f, 1.f};
                if (whole) lds_load_vec<4>(wv + 16 * ks + 4 * lg, w4);
                const u32x2 d = *reinterpret_cast<const u32x2*>(dT + (wave * 16 + lr) * kStride + 8 * ks + 2 * lg);
                uint32_t h[4], lo[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = w4[r] * half_to_f32<IO>((d[r >> 1] >> ((r & 1) * 16)) & 0xffffu);
                    split2<IO>(x, h[r], lo[r]);
                }
                const u32x2 bhi = __builtin_bit_cast(u32x2, __builtin_bit_cast(uint64_t, u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)}) & keep[ks]);
                const u32x2 blo = __builtin_bit_cast(u32x2, __builtin_bit_cast(uint64_t, u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)}) & keep[ks]);
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const u32x2 a0 = *reinterpret_cast<const u32x2*>(kT + (16 * i + lr) * kStride + 8 * ks + 2 * lg);
                    const u32x2 a = __builtin_bit_cast(u32x2, __builtin_bit_cast(uint64_t, a0) & keep[ks]);
                    acc[i] = mfma16<IO>(a, bhi, acc[i]);
                    acc[i] = mfma16<IO>(a, blo, acc[i]);
                }
            }
            if (whole) break;
        }
        __syncthreads();                                      // LDS is restaged next
    };
    auto none = [] {};
    if (steps <= kPos) {
        if (steps > 0) load_chunk(0);
        load_state();
        // vmcnt(NI): the chunk is in, the NI state loads may be pending
        __builtin_amdgcn_s_waitcnt((NI & 15) | ((NI >> 4) << 14) | (0x7 << 4) | (0xF << 8));
        if (steps > 0) chunk(0, none);
    } else {
        load_chunk(0);
        uint32_t t0 = 0;
        for (; t0 + kPos < steps; t0 += kPos) chunk(t0, [&] { load_chunk(t0 + kPos); });
        chunk(t0, load_state);
    }


    // U: accumulator layout -> LDS -> row layout; S = Gamma * S0 + U -> HBM
    // (or S = acc once the snapshot has been folded in)
#pragma unroll
    for (int i = 0; i < NI; ++i)
        *reinterpret_cast<f32x4*>(frag_lds(i)) = f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const f32x4 uu = *reinterpret_cast<const f32x4*>(piece_lds(u));
        const f32x4 r = absorbed ? uu
                                 : f32x4{fmaf(Gamma, sreg[u].x, uu.x), fmaf(Gamma, sreg[u].y, uu.y),
                                         fmaf(Gamma, sreg[u].z, uu.z), fmaf(Gamma, sreg[u].w, uu.w)};
        stream_store(r, reinterpret_cast<f32x4*>(sout + (l + 64 * u) * 4));
    }
}

template <int IO, int DK, int NW>
hipError_t launch_nw(const ReplayArgs& a, hipStream_t stream) {
    constexpr uint32_t rows = 16u * NW;
    const uint32_t slices = a.Dv / rows;
    const uint64_t grid = static_cast<uint64_t>(a.B) * a.Hv * slices;
    if (a.mask != nullptr)
        hipLaunchKernelGGL((gdn_replay_mfma_kernel<IO, DK, NW, true>), dim3(static_cast<uint32_t>(grid)),
                           dim3(64 * NW), 0, stream, a.delta_log, a.k_log, a.g_log, a.state_in, a.mask,
                           a.state_out, a.T_log, a.Hv, a.Dv, slices, a.steps);
    else
        hipLaunchKernelGGL((gdn_replay_mfma_kernel<IO, DK, NW, false>), dim3(static_cast<uint32_t>(grid)),
                           dim3(64 * NW), 0, stream, a.delta_log, a.k_log, a.g_log, a.state_in, a.mask,
                           a.state_out, a.T_log, a.Hv, a.Dv, slices, a.steps);
    return hipGetLastError();
}

// Four waves (64 value rows) per workgroup, unless the caller chose two.
template <int IO, int DK>
hipError_t launch_dk(const ReplayArgs& a, hipStream_t stream) {
    if (a.matrix_waves == 2) return launch_nw<IO, DK, 2>(a, stream);
    return launch_nw<IO, DK, 4>(a, stream);
}

template <int IO>
hipError_t launch_io(const ReplayArgs& a, hipStream_t stream) {
    switch (a.Dk) {
        case 32: return launch_dk<IO, 32>(a, stream);
        case 64: return launch_dk<IO, 64>(a, stream);
        case 128: return launch_dk<IO, 128>(a, stream);
        case 192: return launch_dk<IO, 192>(a, stream);
        case 256: return launch_dk<IO, 256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool replay_mfma_possible(const ReplayArgs& a) {
    if (a.io != kF16 && a.io != kBF16) return false;
    if (a.Dv % 64 != 0) return false;                         // whole 64-row workgroups
    // four work-items per state row (64 per 16-row wave), 2^32 - 1 at most per launch
    return static_cast<uint64_t>(a.B) * a.Hv * a.Dv * 4 <= 0xffffffffull;
}

bool replay_mfma_applies(const ReplayArgs& a) {
    if (a.fold == kFoldValu || !replay_mfma_possible(a)) return false;
    return a.fold == kFoldMatrix || a.steps >= kReplayMfmaFromSteps;
}

hipError_t launch_replay_mfma(const ReplayArgs& a, hipStream_t stream) {
    return a.io == kF16 ? launch_io<kF16>(a, stream) : launch_io<kBF16>(a, stream);
}

}  // namespace gdn
