// gdn_record for short tapes (2 to 4 steps) of bf16 I/O, the speculative-
// decode case, with its dense products on the matrix cores, gfx950.
//
// What it computes is the record kernel (macro `gated_delta_record!`) of the
// metaltile-std 0.1.0 page src/ffai/gated_delta_replay.rs, the same outputs
// as gdn_record.hip (y, the tape delta_log, the final state and the optional
// k_log / g_log capture); only the order of the arithmetic differs.
//
// Over a tape of T steps starting from state S0 (rows dv, columns dk), with
// inactive steps taken as identity steps (g = 1, beta = 0, k = q = 0, and
// nothing written), let
//     gamma_t = g_0 ... g_t,   M[t,s] = g_{s+1} ... g_t  (s < t),  M[t,t] = 1,
//     G[t,s] = k_t . k_s,      H[t,s] = q_t . k_s,
//     XK[t] = S0 k_t,          XQ[t] = S0 q_t   (one value per state row).
// Unrolling the recurrence, the step-t read-out of the decayed row is
//     kv_t = gamma_t XK[t] + sum_{s<t} M[t,s] G[t,s] delta_s,
// so delta_t = beta_t (v_t - kv_t) row by row in step order, then
//     y_t  = gamma_t XQ[t] + sum_{s<=t} M[t,s] H[t,s] delta_s,
//     S_T  = gamma_{T-1} S0 + sum_s M[T-1,s] delta_s k_s^T.
// [XK XQ] = S0 [K; Q]^T is a [Dv x Dk] x [Dk x 2T] product and the last line a
// rank-T update of the [Dv x Dk] state: the two dense contractions run on the
// matrix cores (v_mfma_f32_16x16x32_bf16 for X and G / H, 16x16x16 for the
// update), and what is left on the VALU per state row is the short
// triangular recurrence above.  In the per-step form every step costs four
// VALU operations per state value; here the state is touched by the VALU
// only to split it into matrix-core operands and to scale it by gamma.
//
// Precision.  Keys and queries are bf16 and enter exactly.  The state and
// rho_s delta_s enter as hi + lo, two bf16 numbers with hi = round(x) and
// lo = round(x - hi) (about 16 significant bits); accumulation is fp32.
//
// Mapping.  One wave per workgroup takes 16 consecutive value rows of one
// head (one-wave workgroups start and finish independently, which overlaps
// one workgroup's memory traffic with another's arithmetic better than
// larger workgroups sharing a barrier).  The keys and queries of the steps
// (and the keys transposed) are staged in LDS; every input of the call is
// loaded right after the state, in one round trip.  Why not the per-step
// VALU form: at 4 steps it issues about 750 vector instructions per wave
// (four per state value and step, plus reductions and conversions), which
// left the speculative-decode record issue-bound.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int kSteps = 4;              // longest tape this kernel takes
constexpr int kWaveRows = 16;          // value rows per wave

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// D += A B, 16 x 16 x 32 bf16: lane l gives row l % 16 of A and column
// l % 16 of B over the eight sum positions 8 (l / 16) .. +7 (as long as A and
// B use the same positions for a lane group, which eight does not matter).
__device__ __forceinline__ f32x4v mfma_k32(u32x4 a, u32x4 b, f32x4v acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   acc, 0, 0, 0);
}

// D += A B, 16 x 16 x 16 bf16: lane l gives row l % 16 of A and column l % 16
// of B over the sum positions 4 (l / 16) .. +3.  D[4 (l / 16) + r][l % 16]
// comes back in lane l, r = 0..3 (both instructions).
__device__ __forceinline__ f32x4v mfma_k16(u32x2 a, u32x2 b, f32x4v acc) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b),
                                                     acc, 0, 0, 0);
}

// Two floats rounded to nearest-even bf16 and packed, the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2v));
}

// x = hi + lo in bf16 for two floats at once (packed like pack_bf16).
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16(a, b);
    lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// LDS of one workgroup (one wave): the staged keys and queries of the steps
// (rows 0..3 keys, 4..7 queries, inactive or absent steps as zero rows), the
// keys transposed ([dk][step], 8 bytes a column), and the wave's 16 state
// rows, through which the state changes layout.
template <int DK>
struct RecordMfmaLds {
    static constexpr int KQROW = DK * 2 + 16;              // one bf16 key or query row, padded
    static constexpr int KQ = 0;
    static constexpr int KT = KQ + 2 * kSteps * KQROW;
    static constexpr int SROW = DK * 4 + 16;               // one fp32 state row, padded (bytes)
    static constexpr int STATE = KT + DK * kSteps * 2;
    static constexpr int BYTES = STATE + 16 * SROW;
};

// One wave per workgroup, 16 consecutive value rows of one head.
//
// Layout.  Lane l works on state row lr = l % 16 and, within every 16-column
// tile i of the row, on the four columns 16 i + 4 lg .. +3 (lg = l / 16):
// exactly the lane's part of the 16 x 16 accumulator tile of S^T that the
// update produces.  The X product's 32-deep steps are ordered to match: step
// s sums over columns {16 (2s) + 4 lg .. +3} u {16 (2s + 1) + 4 lg .. +3} for
// lane group lg (any eight columns serve, as long as A and B agree), so the
// state values a lane feeds the matrix cores are the ones it scales by gamma
// and accumulates into: one read of the state serves both.  ROWS_IN: the
// state comes in row by row (whole 128-byte lines per instruction) and moves
// into that layout through LDS; otherwise each lane loads its 16-byte pieces
// straight from memory (half lines per instruction, but no LDS round trip:
// faster while every workgroup of the launch is resident at once, slower
// once the launch streams).  The result always leaves row by row, through
// LDS (stores of half lines cost more than the round trip).
template <int DK, bool ROWS_IN>
__global__ __launch_bounds__(64) void gdn_record_mfma_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ g, const void* __restrict__ beta,
    const float* state_in, const uint32_t* __restrict__ mask,
    void* __restrict__ y, float* state_out, void* __restrict__ delta_log,
    void* __restrict__ k_log, void* __restrict__ g_log,
    uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dv, uint32_t slices, int tiled)
{
    using Lds = RecordMfmaLds<DK>;
    constexpr int NI = DK / 16;            // column tiles: 16-byte state pieces per lane
    constexpr int KSTEPS = DK / 32;        // 32-deep steps of the X product
    constexpr int RP = DK / 8;             // 16-byte pieces of one bf16 key or query row
    constexpr int KQP = 2 * kSteps * RP;   // pieces of the staged keys and queries
    constexpr int KQJ = (KQP + 63) / 64;   // staged pieces per lane

    const uint32_t l = threadIdx.x;
    const uint32_t lr = l & 15u, lg = l >> 4;

    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const uint32_t n = blk / slices;                           // b * Hv + hv
    const uint32_t dv0 = (blk - n * slices) * kWaveRows;
    const uint32_t b = n / Hv;
    const uint32_t hv = n - b * Hv;
    const uint32_t hk = tiled ? hv % Hk : hv / (Hv / Hk);
    const uint32_t row = dv0 + lr;                             // this lane's state row in the head

    __shared__ __align__(16) unsigned char lds[Lds::BYTES];

    // ---- every load of the call, state first
    const float* sin = state_in + (static_cast<size_t>(n) * Dv + dv0) * DK;
    float* sout = state_out + (static_cast<size_t>(n) * Dv + dv0) * DK;
    f32x4 sreg[NI];        // ROWS_IN: piece l + 64 i of the rows; else tile i's piece of row lr
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const size_t off = ROWS_IN ? (l + 64u * i) * 4 : lr * DK + 16 * i + 4 * lg;
        sreg[i] = stream_load(reinterpret_cast<const f32x4*>(sin + off));
    }

    // staged key / query pieces of this lane, piece p = l + 64 j: which (0
    // keys, 1 queries), step st (clamped to the tape for the load), eight
    // columns from pc * 8
    u32x4 kqraw[KQJ];
#pragma unroll
    for (int j = 0; j < KQJ; ++j) {
        const uint32_t p = l + 64u * j;
        const uint32_t which = p / (kSteps * RP), st = (p / RP) % kSteps, pc = p % RP;
        const uint32_t stc = st < T ? st : T - 1;
        kqraw[j] = u32x4{0u, 0u, 0u, 0u};
        if (p < static_cast<uint32_t>(KQP)) {
            const uint16_t* src = static_cast<const uint16_t*>(which == 0 ? k : q);
            kqraw[j] = *reinterpret_cast<const u32x4*>(src + ((static_cast<size_t>(b) * T + stc) * Hk + hk) * DK +
                                                       pc * 8);
        }
    }
    uint32_t vraw[kSteps], graw[kSteps], braw[kSteps], mk[kSteps];
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
        const uint32_t tc = static_cast<uint32_t>(t) < T ? static_cast<uint32_t>(t) : T - 1;
        const size_t bt = static_cast<size_t>(b) * T + tc;
        vraw[t] = static_cast<const uint16_t*>(v)[(bt * Hv + hv) * Dv + row];
        graw[t] = static_cast<const uint16_t*>(g)[bt * Hv + hv];
        braw[t] = static_cast<const uint16_t*>(beta)[bt * Hv + hv];
        mk[t] = mask != nullptr ? mask[bt] : 1u;
    }
    bool act[kSteps];                                          // uniform over the workgroup
#pragma unroll
    for (int t = 0; t < kSteps; ++t) act[t] = static_cast<uint32_t>(t) < T && mk[t] != 0u;

    // ---- staging: keys and queries (zero rows for inactive or absent steps)
    // and the keys transposed; the tape capture
#pragma unroll
    for (int j = 0; j < KQJ; ++j) {
        const uint32_t p = l + 64u * j;
        if (p >= static_cast<uint32_t>(KQP)) continue;
        const uint32_t which = p / (kSteps * RP), st = (p / RP) % kSteps, pc = p % RP;
        bool a = act[0];
#pragma unroll
        for (int t = 1; t < kSteps; ++t) a = st == static_cast<uint32_t>(t) ? act[t] : a;
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 val = a ? kqraw[j] : z;
        *reinterpret_cast<u32x4*>(lds + Lds::KQ + (which * kSteps + st) * Lds::KQROW + pc * 16) = val;
        if (which == 0) {
            uint16_t* kt = reinterpret_cast<uint16_t*>(lds + Lds::KT);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                kt[(pc * 8 + e) * kSteps + st] = static_cast<uint16_t>(val[e >> 1] >> ((e & 1) * 16));
            if (a && dv0 == 0 && k_log != nullptr)             // tape capture: bit copies
                *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(k_log) +
                                          ((static_cast<size_t>(b) * T + st) * Hv + hv) * DK + pc * 8) = kqraw[j];
        }
    }
    if (dv0 == 0 && g_log != nullptr && l < static_cast<uint32_t>(kSteps)) {
        uint32_t gb = graw[0];
        bool a = act[0];
#pragma unroll
        for (int t = 1; t < kSteps; ++t) {
            gb = l == static_cast<uint32_t>(t) ? graw[t] : gb;
            a = l == static_cast<uint32_t>(t) ? act[t] : a;
        }
        if (a) static_cast<uint16_t*>(g_log)[(static_cast<size_t>(b) * T + l) * Hv + hv] = static_cast<uint16_t>(gb);
    }
    unsigned char* sbuf = lds + Lds::STATE;
    if constexpr (ROWS_IN) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int p = static_cast<int>(l) + 64 * i;
            *reinterpret_cast<f32x4*>(sbuf + (p / (DK / 4)) * Lds::SROW + (p % (DK / 4)) * 16) = sreg[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NI; ++i)
            sreg[i] = *reinterpret_cast<const f32x4*>(sbuf + lr * Lds::SROW + (16 * i + 4 * lg) * 4);
    } else {
        __syncthreads();
    }

    // ---- X = [K; Q] S0^T and the Gram products [K; Q] K^T, step s over the
    // columns of tiles 2s and 2s + 1 (this lane's four of each)
    f32x4v x = {0.f, 0.f, 0.f, 0.f}, gh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const unsigned char* kq = lds + Lds::KQ + (lr & 7u) * Lds::KQROW;
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(kq + (16 * (2 * s) + 4 * lg) * 2);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(kq + (16 * (2 * s + 1) + 4 * lg) * 2);
        u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
        a = lr < 2u * kSteps ? a : z;
        const f32x4 s0 = sreg[2 * s], s1 = sreg[2 * s + 1];
        uint32_t h[4], o[4];
        split_pair(s0.x, s0.y, h[0], o[0]);
        split_pair(s0.z, s0.w, h[1], o[1]);
        split_pair(s1.x, s1.y, h[2], o[2]);
        split_pair(s1.z, s1.w, h[3], o[3]);
        const u32x4 hi = {h[0], h[1], h[2], h[3]}, lo = {o[0], o[1], o[2], o[3]};
        x = mfma_k32(a, hi, x);
        x = mfma_k32(a, lo, x);
        gh = mfma_k32(a, lr < static_cast<uint32_t>(kSteps) ? a : z, gh);
    }
    // lane l now holds X[4 lg + r][row lr]: XK[r] for lg = 0, XQ[r] for lg = 1;
    // and G[r][lr] (lg = 0), H[r][lr] (lg = 1) for lr < kSteps.

    // ---- the per-row recurrence (every lane for its row lr; the uniform
    // coefficients from lanes 0..3 and 16..19)
    float gt[kSteps], bt_[kSteps], vt[kSteps];
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
        gt[t] = act[t] ? bf16_bits_to_f32(graw[t]) : 1.f;
        bt_[t] = bf16_bits_to_f32(braw[t]);
        vt[t] = bf16_bits_to_f32(vraw[t]);
    }
    float xk[kSteps], xq[kSteps];
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
        xk[t] = __shfl(x[t], static_cast<int>(lr), 64);
        xq[t] = __shfl(x[t], static_cast<int>(lr + 16), 64);
    }
    float G[kSteps][kSteps], H[kSteps][kSteps];
#pragma unroll
    for (int t = 0; t < kSteps; ++t)
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            G[t][s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gh[t]), s));
            H[t][s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gh[t]), 16 + s));
        }
    float gam[kSteps], M[kSteps][kSteps];
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
        gam[t] = t == 0 ? gt[0] : gam[t - 1] * gt[t];
        M[t][t] = 1.f;
#pragma unroll
        for (int s = t - 1; s >= 0; --s) M[t][s] = M[t][s + 1] * gt[s + 1];
    }
    float dl[kSteps], yo[kSteps];
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
        float kv = gam[t] * xk[t];
#pragma unroll
        for (int s = 0; s < t; ++s) kv = fmaf(M[t][s] * G[t][s], dl[s], kv);
        dl[t] = act[t] ? (vt[t] - kv) * bt_[t] : 0.f;
        float yy = gam[t] * xq[t];
#pragma unroll
        for (int s = 0; s <= t; ++s) yy = fmaf(M[t][s] * H[t][s], dl[s], yy);
        yo[t] = yy;
    }
    if (lg == 0u) {
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
            if (!act[t]) continue;
            const size_t o = ((static_cast<size_t>(b) * T + t) * Hv + hv) * Dv + row;
            static_cast<uint16_t*>(y)[o] = static_cast<uint16_t>(f32_to_bf16_bits(yo[t]));
            if (delta_log != nullptr)
                static_cast<uint16_t*>(delta_log)[o] = static_cast<uint16_t>(f32_to_bf16_bits(dl[t]));
        }
    }

    // ---- S_T^T = gamma_{T-1} S0^T + K^T (rho o Delta), tile i = columns 16 i ..
    // A: column 16 i + lr of K^T over the steps (lanes lg = 0; zero elsewhere);
    // B: rho_s delta_s of row lr (lanes lg = 0) as hi + lo.  Lane l's tile-i
    // result is row lr, columns 16 i + 4 lg .. +3: stored as it stands.
    const float gT = gam[kSteps - 1];
    u32x2 bhi = {0u, 0u}, blo = {0u, 0u};
    if (lg == 0u) {
        float r[kSteps];
#pragma unroll
        for (int s = 0; s < kSteps; ++s) r[s] = M[kSteps - 1][s] * dl[s];
        uint32_t h0, h1, o0, o1;
        split_pair(r[0], r[1], h0, o0);
        split_pair(r[2], r[3], h1, o1);
        bhi = u32x2{h0, h1};
        blo = u32x2{o0, o1};
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        f32x4v acc = {gT * sreg[i].x, gT * sreg[i].y, gT * sreg[i].z, gT * sreg[i].w};
        u32x2 a = *reinterpret_cast<const u32x2*>(lds + Lds::KT + (16 * i + lr) * kSteps * 2);
        const u32x2 z = {0u, 0u};
        a = lg == 0u ? a : z;
        acc = mfma_k16(a, bhi, acc);
        acc = mfma_k16(a, blo, acc);
        sreg[i] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    }
    if constexpr (ROWS_IN) __syncthreads();                    // every read of the staged rows is done
#pragma unroll
    for (int i = 0; i < NI; ++i)
        *reinterpret_cast<f32x4*>(sbuf + lr * Lds::SROW + (16 * i + 4 * lg) * 4) = sreg[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int p = static_cast<int>(l) + 64 * i;
        const f32x4 r = *reinterpret_cast<const f32x4*>(sbuf + (p / (DK / 4)) * Lds::SROW + (p % (DK / 4)) * 16);
        stream_store(r, reinterpret_cast<f32x4*>(sout + (l + 64u * i) * 4));
    }
}

template <int DK, bool ROWS_IN>
hipError_t launch_cfg(const RecordArgs& a, uint32_t slices, uint64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((gdn_record_mfma_kernel<DK, ROWS_IN>), dim3(static_cast<uint32_t>(grid)), dim3(64), 0, stream,
                       a.q, a.k, a.v, a.g, a.beta, a.state_in, a.mask, a.y, a.state_out, a.delta_log, a.k_log,
                       a.g_log, a.T, a.Hk, a.Hv, a.Dv, slices, a.map);
    return hipGetLastError();
}

// Workgroups per CU up to which the whole launch is taken to be resident at
// once (the kernel holds about 14 one-wave workgroups per CU): the
// state then comes straight in, half lines and all (8.9 against 9.4 us for
// a record of 4 steps at batch 8 over 32 heads of 128 x 128); past that the
// launch streams and full-line loads pay (54 against 67 us at batch 64).
constexpr uint64_t kResidentPerCu = 16;

template <int DK>
hipError_t launch_dk(const RecordArgs& a, hipStream_t stream) {
    const uint32_t slices = a.Dv / kWaveRows;
    const uint64_t grid = static_cast<uint64_t>(a.B) * a.Hv * slices;
    if (grid <= kResidentPerCu * compute_units()) return launch_cfg<DK, false>(a, slices, grid, stream);
    return launch_cfg<DK, true>(a, slices, grid, stream);
}

}  // namespace

bool record_mfma_applies(const RecordArgs& a) {
    if (a.forced.rows_per_thread != 0) return false;           // a forced tiling runs the VALU kernels
    if (a.io != kBF16 || a.T < 2 || a.T > static_cast<uint32_t>(kSteps)) return false;
    if (a.Dv % kWaveRows != 0 || !(a.Dk == 32 || a.Dk == 64 || a.Dk == 128 || a.Dk == 192)) return false;
    // four work-items per state row, at most 2^32 - 1 per launch
    return static_cast<uint64_t>(a.B) * a.Hv * a.Dv * 4 <= 0xffffffffull;
}

hipError_t launch_record_mfma(const RecordArgs& a, hipStream_t stream) {
    switch (a.Dk) {
        case 32: return launch_dk<32>(a, stream);
        case 64: return launch_dk<64>(a, stream);
        case 128: return launch_dk<128>(a, stream);
        case 192: return launch_dk<192>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
