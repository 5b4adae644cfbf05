// gdn_prefill: the record step over a long sequence (a prefill), computed a
// chunk of 64 steps at a time as dense contractions on the matrix cores, gfx950.
//
// What it computes is exactly the record kernel (macro `gated_delta_record!`)
// of the metaltile-std 0.1.0 page src/ffai/gated_delta_replay.rs, the same
// quantities as gdn_record.hip (y, the innovation tape delta_log and the final
// state); only the order of the arithmetic differs.  The mlx-native 0.6.5 page
// mlx_native/ops/repeat_tiled.rs names this caller ("chunk-prefill") but gives
// no algorithm for it; the chunk form below is derived from the per-step
// recurrence alone.
//
// Chunk form.  Take a chunk of C = 64 steps starting from state S0 (rows dv,
// columns dk).  An inactive step (masked, or past T) is the identity step
// g = 1, beta = 0 with k = q = v = 0.  With
//     gamma_t = g_0 ... g_t,   M[t,s] = g_{s+1} ... g_t  (s <= t, else 0),
//     G[t,s]  = k_t . k_s,     H[t,s] = q_t . k_s,
// the record step t reads kv_t = g_t S_{t-1} k_t
//     = gamma_t S0 k_t + sum_{s<t} M[t,s] G[t,s] delta_s,
// so the innovations of the chunk solve a unit lower-triangular system
//     (I + A) Delta = diag(beta) R,   A[t,s] = beta_t M[t,s] G[t,s]  (s < t),
//     R_t = v_t - gamma_t S0 k_t,
// i.e. Delta = Tb R with Tb = (I + A)^-1 diag(beta).  Then
//     y_t  = S_t q_t = gamma_t S0 q_t + sum_{s<=t} M[t,s] H[t,s] delta_s,
//     S_C  = gamma_63 S0 + sum_s M[63,s] delta_s k_s^T.
// Tb and P = M o H depend on the chunk's keys, queries and gates only, so a
// first kernel (prep) forms them for every chunk in parallel; a second kernel
// (scan) carries the state through the chunks in order, with every product a
// 16x16x16 MFMA: X = [K; Q] S0^T, Delta = Tb R, Y = gamma o XQ + P Delta and
// S^T <- gamma_63 S^T + K^T (rho o Delta), rho_s = M[63,s].
//
// Precision.  Keys and queries are bf16 and enter the MFMAs exactly.  Every
// fp32 operand (the state, R, Delta, Tb, P) enters as hi + lo, two bf16 numbers
// with hi = round(x) and lo = round(x - hi) (about 16 significant bits); an
// fp32 x fp32 product takes three MFMAs (hi.hi + hi.lo + lo.hi), a bf16 x fp32
// product two.  Accumulation is fp32.  M is formed by running products of the
// gates (no division), so zero or tiny gates are exact.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int kC = 64;            // steps per chunk
constexpr int kDk = 128;          // key width this path is built for
constexpr int kRows = 16;         // state rows per scan workgroup

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// acc += A (16 x 16) * B (16 x 16) with bf16 operands.  Lane l holds
// A[l % 16][4 (l / 16) + 0..3], B[4 (l / 16) + 0..3][l % 16] and returns
// D[4 (l / 16) + r][l % 16], r = 0..3.
__device__ __forceinline__ f32x4v mfma_bf16(u32x2 a, u32x2 b, f32x4v acc) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), acc, 0, 0, 0);
}

// Two floats rounded to nearest-even bf16 and packed (v_cvt_pk_bf16_f32),
// the first in the low half.  Used only for the internal hi/lo operands.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2v));
}

// x = hi + lo in bf16, for four values at once (fragment order kept).
__device__ __forceinline__ void split4(const f32x4v& x, u32x2& hi, u32x2& lo) {
    hi.x = cvt_pk_bf16(x[0], x[1]);
    hi.y = cvt_pk_bf16(x[2], x[3]);
    lo.x = cvt_pk_bf16(x[0] - __uint_as_float(hi.x << 16), x[1] - __uint_as_float(hi.x & 0xffff0000u));
    lo.y = cvt_pk_bf16(x[2] - __uint_as_float(hi.y << 16), x[3] - __uint_as_float(hi.y & 0xffff0000u));
}

__device__ __forceinline__ void split1(float x, uint16_t& hi, uint16_t& lo) {
    const uint32_t h = cvt_pk_bf16(x, 0.0f) & 0xffffu;
    hi = static_cast<uint16_t>(h);
    lo = static_cast<uint16_t>(cvt_pk_bf16(x - bf16_bits_to_f32(h), 0.0f));
}

__device__ __forceinline__ u32x2 zero2() {
    u32x2 z;
    z.x = 0u;
    z.y = 0u;
    return z;
}

__device__ __forceinline__ u32x2 load8(const void* base, size_t byte_off) {
    return *reinterpret_cast<const u32x2*>(static_cast<const char*>(base) + byte_off);
}

__device__ __forceinline__ bool step_active(const uint32_t* mask, uint32_t b, uint32_t T, uint32_t t) {
    return t < T && (mask == nullptr || mask[static_cast<size_t>(b) * T + t] > 0u);
}

}  // namespace

// Per (b, hv, chunk) block of the workspace, written by prep and read by scan.
struct PrefillWs {
    static constexpr int kMat = kC * kC * 2;             // one 64 x 64 bf16 matrix
    static constexpr int kTbHi = 0, kTbLo = kMat, kPHi = 2 * kMat, kPLo = 3 * kMat;
    static constexpr int kGamma = 4 * kMat;              // gamma_t, fp32 [64]
    static constexpr int kRho = kGamma + kC * 4;         // rho_t = M[63, t], fp32 [64]
    static constexpr int kBytes = kRho + kC * 4;         // 33280
};

namespace {

// Row I of the forward substitution (I + A) T = identity, then the rows after
// it.  Four consecutive lanes share column c of T; lane q of the four keeps
// col[j] for j = 4m + q in mine[m] and sums the terms of those j, and a quad
// reduction gives every lane of the four the whole sum.  A is read from LDS
// in the layout Aq[(i * 4 + q) * kAqRow + m] = A[i, 4m + q], so one 16-byte
// read covers four of a lane's terms (the same address for every column).
// Entries of A at and above the diagonal are stored zeros, and mine[] of rows
// not yet reached is zero, so the sums need no masks.  Row indices are
// template parameters so that mine[] stays in registers.
constexpr int kAqRow = 20;       // floats per (row, q): 16 used, padded

template <int I>
__device__ __forceinline__ void forward_quad_row(float (&mine)[16], const float* Aq, int c, int q) {
    constexpr int NM = (I + 3) / 4;                 // m with 4m + q < I for some q
    const float* row = Aq + (I * 4 + q) * kAqRow;
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int m4 = 0; m4 < (NM + 3) / 4; ++m4) {
        const float4 a = *reinterpret_cast<const float4*>(row + 4 * m4);
        if (4 * m4 + 0 < NM) p0 = fmaf(a.x, mine[4 * m4 + 0], p0);
        if (4 * m4 + 1 < NM) p1 = fmaf(a.y, mine[4 * m4 + 1], p1);
        if (4 * m4 + 2 < NM) p0 = fmaf(a.z, mine[4 * m4 + 2], p0);
        if (4 * m4 + 3 < NM) p1 = fmaf(a.w, mine[4 * m4 + 3], p1);
    }
    float part = p0 + p1;
    part += dpp_read<0xb1>(part);      // quad_perm [1,0,3,2]
    part += dpp_read<0x4e>(part);      // quad_perm [2,3,0,1]: the same bits on all four lanes
    const float val = (I == c ? 1.0f : 0.0f) - part;
    mine[I >> 2] = (I & 3) == q ? val : mine[I >> 2];
    if constexpr (I + 1 < kC) forward_quad_row<I + 1>(mine, Aq, c, q);
}

// ------------------------------------------------------------------ prep
//
// One workgroup of four waves per (b, hv, chunk).  Wave w owns row tile w
// (steps 16w .. 16w+15) of the 64 x 64 matrices.
template <int IO>
__global__ __launch_bounds__(256) void gdn_prefill_prep_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ g,
    const void* __restrict__ beta, const uint32_t* __restrict__ mask,
    unsigned char* __restrict__ ws, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t nchunks,
    uint32_t group, int tiled)
{
    static_assert(IO == kBF16, "the chunked prefill takes bf16 I/O");
    constexpr int MS = kC + 1;       // row stride of M in floats
    __shared__ __align__(16) float gs[kC];
    __shared__ float bs[kC];
    __shared__ float Ml[kC * MS];
    __shared__ __align__(16) float Aq[kC * 4 * kAqRow];

    const uint32_t tid = threadIdx.x, l = tid & 63u, w = tid >> 6;
    const uint32_t lr = l & 15u, lg = l >> 4;
    const uint32_t n = blockIdx.x / nchunks;               // b * Hv + hv
    const uint32_t c = blockIdx.x - n * nchunks;
    const uint32_t b = n / Hv, hv = n - b * Hv;
    const uint32_t hk = tiled ? hv % Hk : hv / group;
    const uint32_t t0 = c * kC;
    unsigned char* wsb = ws + (static_cast<size_t>(n) * nchunks + c) * PrefillWs::kBytes;

    // Key fragments of all four row tiles, and key and query fragments of
    // this wave's tile: lane holds x[16 tile + lr][16 ks + 4 lg .. +3].  All
    // loads are issued first (steps past T read row T-1); rows of inactive
    // steps are then replaced by zeros (a select, so a NaN there cannot enter
    // a product).
    u32x2 kf[4][kDk / 16], kw[kDk / 16], qf[kDk / 16];
    uint32_t mt[4], mw;
    const size_t kq_row = static_cast<size_t>(Hk) * kDk * 2;   // bytes per step
    const size_t kq_base = (static_cast<size_t>(b) * T * Hk + hk) * kDk * 2 + lg * 8;
#pragma unroll
    for (int tile = 0; tile < 4; ++tile) {
        const uint32_t t = t0 + 16u * tile + lr, tc = t < T ? t : T - 1;
        const size_t off = kq_base + static_cast<size_t>(tc) * kq_row;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) kf[tile][ks] = load8(k, off + ks * 32);
        mt[tile] = mask ? mask[static_cast<size_t>(b) * T + tc] : 1u;
    }
    {
        const uint32_t t = t0 + 16u * w + lr, tc = t < T ? t : T - 1;
        const size_t off = kq_base + static_cast<size_t>(tc) * kq_row;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) {
            kw[ks] = load8(k, off + ks * 32);
            qf[ks] = load8(q, off + ks * 32);
        }
        mw = mask ? mask[static_cast<size_t>(b) * T + tc] : 1u;
    }
    if (tid < kC) {
        const uint32_t t = t0 + tid, tc = t < T ? t : T - 1;
        const size_t i = (static_cast<size_t>(b) * T + tc) * Hv + hv;
        const float gl = io_load1<IO>(g, i), bl = io_load1<IO>(beta, i);
        const uint32_t m = mask ? mask[static_cast<size_t>(b) * T + tc] : 1u;
        const bool act = t < T && m > 0u;
        gs[tid] = act ? gl : 1.0f;
        bs[tid] = act ? bl : 0.0f;
    }
#pragma unroll
    for (int tile = 0; tile < 4; ++tile) {
        const bool act = t0 + 16u * tile + lr < T && mt[tile] > 0u;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) kf[tile][ks] = act ? kf[tile][ks] : zero2();
    }
    {
        const bool act = t0 + 16u * w + lr < T && mw > 0u;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) {
            kw[ks] = act ? kw[ks] : zero2();
            qf[ks] = act ? qf[ks] : zero2();
        }
    }
    __syncthreads();

    // M by running products of the gates (gates held in registers): thread t
    // walks s = 63 .. 0, multiplying in g_s once s <= t.
    if (tid < kC) {
        float gr[kC];
#pragma unroll
        for (int s4 = 0; s4 < kC / 4; ++s4) {
            const float4 v4 = *reinterpret_cast<const float4*>(&gs[4 * s4]);
            gr[4 * s4] = v4.x; gr[4 * s4 + 1] = v4.y; gr[4 * s4 + 2] = v4.z; gr[4 * s4 + 3] = v4.w;
        }
        const int t = static_cast<int>(tid);
        float p = 1.0f;
#pragma unroll
        for (int s = kC - 1; s >= 0; --s) {
            Ml[t * MS + s] = s <= t ? p : 0.0f;
            p = s <= t ? p * gr[s] : p;
        }
        reinterpret_cast<float*>(wsb + PrefillWs::kGamma)[t] = p;   // gamma_t = g_0 .. g_t
    }
    __syncthreads();
    if (tid < kC) reinterpret_cast<float*>(wsb + PrefillWs::kRho)[tid] = Ml[(kC - 1) * MS + tid];

    // Gram tiles G = K K^T and H = Q K^T of row tile w (all four column tiles;
    // above the diagonal the s <= t masks below make A and P exact zeros).
    // Products of bf16 values are exact in fp32.
    uint16_t* phi = reinterpret_cast<uint16_t*>(wsb + PrefillWs::kPHi);
    uint16_t* plo = reinterpret_cast<uint16_t*>(wsb + PrefillWs::kPLo);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        f32x4v G = {0.f, 0.f, 0.f, 0.f}, H = {0.f, 0.f, 0.f, 0.f};
        f32x4v G2 = G, H2 = H;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ks += 2) {
            G = mfma_bf16(kw[ks], kf[st][ks], G);
            G2 = mfma_bf16(kw[ks + 1], kf[st][ks + 1], G2);
            H = mfma_bf16(qf[ks], kf[st][ks], H);
            H2 = mfma_bf16(qf[ks + 1], kf[st][ks + 1], H2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * static_cast<int>(w) + 4 * static_cast<int>(lg) + r;
            const int s = 16 * st + static_cast<int>(lr);
            const float m = Ml[t * MS + s];
            Aq[(t * 4 + (s & 3)) * kAqRow + (s >> 2)] = s < t ? bs[t] * (m * (G[r] + G2[r])) : 0.0f;
            uint16_t hi, lo;
            split1(s <= t ? m * (H[r] + H2[r]) : 0.0f, hi, lo);
            phi[t * kC + s] = hi;
            plo[t * kC + s] = lo;
        }
    }
    __syncthreads();

    // (I + A)^-1 by forward substitution over all four waves (four lanes per
    // column), then Tb = (I + A)^-1 diag(beta).
    {
        const int col = static_cast<int>(tid >> 2), qq = static_cast<int>(tid & 3u);
        float mine[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) mine[m] = 0.0f;
        forward_quad_row<0>(mine, Aq, col, qq);
        const float bc = bs[col];
        uint16_t* thi = reinterpret_cast<uint16_t*>(wsb + PrefillWs::kTbHi);
        uint16_t* tlo = reinterpret_cast<uint16_t*>(wsb + PrefillWs::kTbLo);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int i = 4 * m + qq;
            uint16_t hi, lo;
            split1(mine[m] * bc, hi, lo);
            thi[i * kC + col] = hi;
            tlo[i * kC + col] = lo;
        }
    }
}

// ------------------------------------------------------------------ scan
//
// One workgroup of eight waves per (b, hv, 16 consecutive value rows).  The
// state is held transposed in MFMA accumulators: wave w owns key columns
// 16w .. 16w+15, lane l holding S[dv0 + l%16][16w + 4 (l/16) + r] -- the
// layout in which the tile is also the B operand of X = K S^T for key step w.
// Waves 0-3 (the K side) take step tile w of the chunk: X_K, R and Delta.
// Waves 4-7 (the Q side) take step tile w-4: X_Q, and Y of the previous chunk
// while the K side solves for Delta (Y is not on the state's dependency chain).
struct ScanIn {
    u32x2 af[kDk / 16];                 // K (K side) or Q (Q side) [16 tt + lr][16 ks + 4 lg ..], as loaded
    u32x2 mh[4], ml[4];                 // Tb (K side) or P (Q side) [16 tt + lr][16 ks + 4 lg ..], hi and lo
    uint32_t vb[4];                     // word holding v at steps 16 tt + 4 lg + r, row lr
    uint32_t mA, mC[4];                 // mask words of those steps (1 without a mask)
    f32x4v gam, rho;                    // gamma, rho at steps 16 tt + 4 lg + r
    float gC;                           // gamma_63
};

// Issue the loads of one chunk.  Nothing here consumes a loaded value, so the
// loads stay in flight while the previous chunk is computed; steps past T
// read step T-1 and are zeroed where the values are used.
__device__ __forceinline__ void scan_load(ScanIn& in, const void* src, const uint32_t* mask,
                                          const void* v, const unsigned char* wsb, int ws_hi,
                                          int ws_lo, uint32_t b, uint32_t hv, uint32_t hk,
                                          uint32_t dv0, uint32_t T, uint32_t Hk, uint32_t Hv,
                                          uint32_t Dv, uint32_t t0, uint32_t tt, uint32_t lr,
                                          uint32_t lg) {
    {
        const uint32_t t = t0 + 16u * tt + lr, tc = t < T ? t : T - 1;
        const size_t off = ((static_cast<size_t>(b) * T + tc) * Hk + hk) * kDk * 2 + lg * 8;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) in.af[ks] = load8(src, off + ks * 32);
        in.mA = mask ? mask[static_cast<size_t>(b) * T + tc] : 1u;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t t = t0 + 16u * tt + 4u * lg + r, tc = t < T ? t : T - 1;
        // The aligned 32-bit word holding the element (Dv is even, so it lies
        // inside v); the half is picked where the value is used.
        const size_t e = ((static_cast<size_t>(b) * T + tc) * Hv + hv) * Dv + dv0 + lr;
        in.vb[r] = static_cast<const uint32_t*>(v)[e >> 1];
        in.mC[r] = mask ? mask[static_cast<size_t>(b) * T + tc] : 1u;
    }
    const size_t frag = ((16u * tt + lr) * kC + 4u * lg) * 2;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        in.mh[ks] = load8(wsb, ws_hi + frag + ks * 32);
        in.ml[ks] = load8(wsb, ws_lo + frag + ks * 32);
    }
    const float* gam = reinterpret_cast<const float*>(wsb + PrefillWs::kGamma);
    const float* rho = reinterpret_cast<const float*>(wsb + PrefillWs::kRho);
    const float4 g4 = *reinterpret_cast<const float4*>(gam + 16u * tt + 4u * lg);
    const float4 r4 = *reinterpret_cast<const float4*>(rho + 16u * tt + 4u * lg);
    in.gam = f32x4v{g4.x, g4.y, g4.z, g4.w};
    in.rho = f32x4v{r4.x, r4.y, r4.z, r4.w};
    in.gC = gam[kC - 1];
}

__device__ __forceinline__ u32x2 lo2(const u32x4& x) { return u32x2{x.x, x.y}; }
__device__ __forceinline__ u32x2 hi2(const u32x4& x) { return u32x2{x.z, x.w}; }

template <int IO>
__global__ __launch_bounds__(512, 1) void gdn_prefill_scan_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* state_in, const uint32_t* __restrict__ mask,
    const unsigned char* __restrict__ ws, void* __restrict__ y, float* state_out,
    void* __restrict__ delta_log, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dv,
    uint32_t nchunks, uint32_t group, int tiled)
{
    static_assert(IO == kBF16, "the chunked prefill takes bf16 I/O");
    constexpr int KTS = kC + 4;                        // K^T row stride in bf16 (136 bytes)
    // Fragments exchanged between the waves: lane-ordered 16-byte (hi, lo) pairs.
    __shared__ __align__(16) u32x4 sfr[kDk / 16][64];  // state, per key step
    __shared__ __align__(16) u32x4 rfr[4][64];         // R, per step tile
    __shared__ __align__(16) u32x4 dfr[2][4][64];      // Delta, two chunks
    __shared__ __align__(16) u32x4 dtf[4][64];         // rho o Delta
    __shared__ __align__(16) uint16_t kt[2][kDk * KTS];   // K^T [dk][t], two chunks

    const uint32_t tid = threadIdx.x, l = tid & 63u, w = tid >> 6;
    const uint32_t lr = l & 15u, lg = l >> 4;
    const uint32_t tt = w & 3u;                         // step tile
    const bool qside = w >= 4u;
    const uint32_t slices = Dv / kRows;
    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const uint32_t n = blk / slices;                    // b * Hv + hv
    const uint32_t dv0 = (blk - n * slices) * kRows;
    const uint32_t b = n / Hv, hv = n - b * Hv;
    const uint32_t hk = tiled ? hv % Hk : hv / group;

    // This lane's 16-byte state piece: row dv0 + lr, columns 16w + 4lg .. +3.
    const size_t srow = (static_cast<size_t>(n) * Dv + dv0 + lr) * kDk + 16u * w + 4u * lg;
    f32x4v acc;
    {
        const float4 s4 = *reinterpret_cast<const float4*>(state_in + srow);
        acc = f32x4v{s4.x, s4.y, s4.z, s4.w};
    }

    const void* src = qside ? q : k;
    const int ws_hi = qside ? PrefillWs::kPHi : PrefillWs::kTbHi;
    const int ws_lo = qside ? PrefillWs::kPLo : PrefillWs::kTbLo;
    void* out = qside ? y : delta_log;                  // what this wave writes (delta_log may be NULL)
    const unsigned char* wsn = ws + static_cast<size_t>(n) * nchunks * PrefillWs::kBytes;
    ScanIn cur, nxt;
    scan_load(nxt, src, mask, v, wsn, ws_hi, ws_lo, b, hv, hk, dv0, T, Hk, Hv, Dv, 0u, tt, lr, lg);

    // One pending output tile per wave (Delta of this chunk on the K side, Y of
    // the previous chunk on the Q side), stored at the start of the next
    // iteration before its prefetch: the prefetched values are then awaited
    // without also waiting for those (conditional, hence uncounted) stores.
    f32x4v pend = {0.f, 0.f, 0.f, 0.f};
    uint32_t pend_act = 0u, pend_t0 = 0u;
    auto flush = [&]() {
        if (out == nullptr) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (pend_act & (1u << r)) {
                const size_t i = ((static_cast<size_t>(b) * T + pend_t0 + 16u * tt + 4u * lg + r) * Hv + hv) * Dv +
                                 dv0 + lr;
                static_cast<uint16_t*>(out)[i] = static_cast<uint16_t>(f32_to_bf16_bits(pend[r]));
            }
        }
        pend_act = 0u;
    };
    // Q side: what Y of a chunk needs one iteration later.
    f32x4v xq_prev = {0.f, 0.f, 0.f, 0.f}, gam_prev = xq_prev;
    u32x2 ph_prev[4], pl_prev[4];
    uint32_t act_prev = 0u;
    auto y_tile = [&](const u32x4 (&dsrc)[4][64]) {
        f32x4v Y, Y2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) Y[r] = gam_prev[r] * xq_prev[r];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4 dd = dsrc[ks][l];
            Y = mfma_bf16(ph_prev[ks], lo2(dd), Y);
            Y2 = mfma_bf16(ph_prev[ks], hi2(dd), Y2);
            Y2 = mfma_bf16(pl_prev[ks], lo2(dd), Y2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) pend[r] = Y[r] + Y2[r];
    };

    for (uint32_t c = 0; c < nchunks; ++c) {
        cur = nxt;
        flush();
        if (c + 1 < nchunks)
            scan_load(nxt, src, mask, v, wsn + (c + 1) * static_cast<size_t>(PrefillWs::kBytes), ws_hi, ws_lo,
                      b, hv, hk, dv0, T, Hk, Hv, Dv, (c + 1) * kC, tt, lr, lg);
        const uint32_t t0 = c * kC;
        uint16_t* ktb = kt[c & 1u];
        // Inactive steps (masked, or past T): zero keys, queries and values.
        {
            const bool a = t0 + 16u * tt + lr < T && cur.mA > 0u;
#pragma unroll
            for (int ks = 0; ks < kDk / 16; ++ks) cur.af[ks] = a ? cur.af[ks] : zero2();
        }
        uint32_t act = 0u;
        f32x4v vv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool a = t0 + 16u * tt + 4u * lg + r < T && cur.mC[r] > 0u;
            vv[r] = a ? bf16_bits_to_f32((cur.vb[r] >> (16u * (lr & 1u))) & 0xffffu) : 0.0f;
            act |= a ? (1u << r) : 0u;
        }

        // State tile -> (hi, lo) fragment for every wave; the K side's key rows,
        // transposed into K^T [dk][t].
        {
            u32x2 hi, lo;
            split4(acc, hi, lo);
            sfr[w][l] = u32x4{hi.x, hi.y, lo.x, lo.y};
        }
        if (!qside) {
#pragma unroll
            for (int ks = 0; ks < kDk / 16; ++ks) {
                const uint32_t dk = 16u * ks + 4u * lg, t = 16u * tt + lr;
                ktb[(dk + 0) * KTS + t] = static_cast<uint16_t>(cur.af[ks].x);
                ktb[(dk + 1) * KTS + t] = static_cast<uint16_t>(cur.af[ks].x >> 16);
                ktb[(dk + 2) * KTS + t] = static_cast<uint16_t>(cur.af[ks].y);
                ktb[(dk + 3) * KTS + t] = static_cast<uint16_t>(cur.af[ks].y >> 16);
            }
        }
        __syncthreads();

        // X = (K or Q) S0^T for step tile tt (hi and lo parts apart).
        f32x4v x = {0.f, 0.f, 0.f, 0.f}, x2 = x;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) {
            const u32x4 sv = sfr[ks][l];
            x = mfma_bf16(cur.af[ks], lo2(sv), x);
            x2 = mfma_bf16(cur.af[ks], hi2(sv), x2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] += x2[r];
        if (!qside) {
            f32x4v R;
#pragma unroll
            for (int r = 0; r < 4; ++r) R[r] = vv[r] - cur.gam[r] * x[r];
            u32x2 hi, lo;
            split4(R, hi, lo);
            rfr[tt][l] = u32x4{hi.x, hi.y, lo.x, lo.y};
        }
        __syncthreads();

        if (!qside) {
            // Delta (step tile tt) = Tb R.  Tb is zero above the diagonal, so
            // the tiles past tt add exact zeros.
            f32x4v D = {0.f, 0.f, 0.f, 0.f}, D2 = D;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4 rr = rfr[ks][l];
                D = mfma_bf16(cur.mh[ks], lo2(rr), D);
                D2 = mfma_bf16(cur.mh[ks], hi2(rr), D2);
                D2 = mfma_bf16(cur.ml[ks], lo2(rr), D2);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) D[r] += D2[r];
            u32x2 hi, lo;
            split4(D, hi, lo);
            dfr[c & 1u][tt][l] = u32x4{hi.x, hi.y, lo.x, lo.y};
            f32x4v Dt;
#pragma unroll
            for (int r = 0; r < 4; ++r) Dt[r] = cur.rho[r] * D[r];
            split4(Dt, hi, lo);
            dtf[tt][l] = u32x4{hi.x, hi.y, lo.x, lo.y};
            pend = D;
            pend_act = act;
            pend_t0 = t0;
        } else if (c > 0) {
            // Y of the previous chunk = gamma o X_Q + P Delta.
            y_tile(dfr[(c - 1) & 1u]);
            pend_act = act_prev;
            pend_t0 = t0 - kC;
        }
        if (qside) {
            xq_prev = x;
            gam_prev = cur.gam;
            act_prev = act;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                ph_prev[ks] = cur.mh[ks];
                pl_prev[ks] = cur.ml[ks];
            }
        }
        __syncthreads();

        // S^T <- gamma_63 S^T + K^T (rho o Delta) for this wave's key tile.
        f32x4v lo_acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= cur.gC;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4 dd = dtf[ks][l];
            const uint32_t dk = 16u * w + lr;
            const u32x2 a = *reinterpret_cast<const u32x2*>(&ktb[dk * KTS + 16 * ks + 4 * lg]);
            acc = mfma_bf16(a, lo2(dd), acc);
            lo_acc = mfma_bf16(a, hi2(dd), lo_acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += lo_acc[r];
    }

    flush();
    if (qside) {
        // Y of the last chunk (its Delta fragments were written before the
        // last iteration's final barrier).
        y_tile(dfr[(nchunks - 1) & 1u]);
        pend_act = act_prev;
        pend_t0 = (nchunks - 1) * kC;
        flush();
    }
    *reinterpret_cast<float4*>(state_out + srow) = make_float4(acc[0], acc[1], acc[2], acc[3]);
}

}  // namespace

size_t prefill_workspace_bytes(uint32_t B, uint32_t T, uint32_t Hv) {
    const size_t nchunks = (static_cast<size_t>(T) + kC - 1) / kC;
    return static_cast<size_t>(B) * Hv * nchunks * PrefillWs::kBytes;
}

bool prefill_supported(uint32_t Dk, uint32_t Dv, int io) {
    return io == kBF16 && Dk == static_cast<uint32_t>(kDk) && Dv % kRows == 0;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    const uint32_t nchunks = (a.T + kC - 1) / kC;
    const uint32_t group = a.Hv / a.Hk;
    const int tiled = a.map == 1;
    auto* ws = static_cast<unsigned char*>(a.workspace);
    hipLaunchKernelGGL(gdn_prefill_prep_kernel<kBF16>, dim3(a.B * a.Hv * nchunks), dim3(256), 0, stream,
                       a.q, a.k, a.g, a.beta, a.mask, ws, a.T, a.Hk, a.Hv, nchunks, group, tiled);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gdn_prefill_scan_kernel<kBF16>, dim3(a.B * a.Hv * (a.Dv / kRows)), dim3(512), 0, stream,
                       a.q, a.k, a.v, a.state_in, a.mask, ws, a.y, a.state_out, a.delta_log, a.T, a.Hk, a.Hv,
                       a.Dv, nchunks, group, tiled);
    return hipGetLastError();
}

}  // namespace gdn
