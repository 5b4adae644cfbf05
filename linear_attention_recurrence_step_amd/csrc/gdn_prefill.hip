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

__device__ __forceinline__ u32x2 pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x2 r;
    r.x = a | (b << 16);
    r.y = c | (d << 16);
    return r;
}

// x = hi + lo in bf16, for four values at once (fragment order kept).
__device__ __forceinline__ void split4(const f32x4v& x, u32x2& hi, u32x2& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        h[r] = f32_to_bf16_bits(x[r]);
        l[r] = f32_to_bf16_bits(x[r] - bf16_bits_to_f32(h[r]));
    }
    hi = pack4(h[0], h[1], h[2], h[3]);
    lo = pack4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ void split1(float x, uint16_t& hi, uint16_t& lo) {
    const uint32_t h = f32_to_bf16_bits(x);
    hi = static_cast<uint16_t>(h);
    lo = static_cast<uint16_t>(f32_to_bf16_bits(x - bf16_bits_to_f32(h)));
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

// Row I of the forward substitution (I + A) T = identity for the column this
// lane owns, then the rows after it.  A is read from LDS (row stride AS, four
// entries per read, the same address for every lane); the row index is a
// template parameter so that col[] stays in registers.
template <int I, int AS>
__device__ __forceinline__ void forward_row(float (&col)[kC], const float* Al, int lane) {
    float acc0 = I == lane ? 1.0f : 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int j4 = 0; j4 < (I + 3) / 4; ++j4) {
        const float4 a = *reinterpret_cast<const float4*>(&Al[I * AS + 4 * j4]);
        if (4 * j4 + 0 < I) acc0 -= a.x * col[4 * j4 + 0];
        if (4 * j4 + 1 < I) acc1 -= a.y * col[4 * j4 + 1];
        if (4 * j4 + 2 < I) acc0 -= a.z * col[4 * j4 + 2];
        if (4 * j4 + 3 < I) acc1 -= a.w * col[4 * j4 + 3];
    }
    col[I] = acc0 + acc1;
    if constexpr (I + 1 < kC) forward_row<I + 1, AS>(col, Al, lane);
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
    constexpr int AS = kC + 4;       // row stride of A in floats (16-byte rows for float4 reads)
    __shared__ float gs[kC], bs[kC];
    __shared__ float Ml[kC * MS];
    __shared__ __align__(16) float Al[kC * AS];

    const uint32_t tid = threadIdx.x, l = tid & 63u, w = tid >> 6;
    const uint32_t lr = l & 15u, lg = l >> 4;
    const uint32_t n = blockIdx.x / nchunks;               // b * Hv + hv
    const uint32_t c = blockIdx.x - n * nchunks;
    const uint32_t b = n / Hv, hv = n - b * Hv;
    const uint32_t hk = tiled ? hv % Hk : hv / group;
    const uint32_t t0 = c * kC;
    unsigned char* wsb = ws + (static_cast<size_t>(n) * nchunks + c) * PrefillWs::kBytes;

    if (tid < kC) {
        const uint32_t t = t0 + tid;
        const bool act = step_active(mask, b, T, t);
        float gv = 1.0f, bv = 0.0f;
        if (t < T) {
            const size_t i = (static_cast<size_t>(b) * T + t) * Hv + hv;
            const float gl = io_load1<IO>(g, i), bl = io_load1<IO>(beta, i);
            gv = act ? gl : 1.0f;
            bv = act ? bl : 0.0f;
        }
        gs[tid] = gv;
        bs[tid] = bv;
    }

    // Key fragments of all four row tiles and query fragments of this wave's
    // tile: lane holds x[16 tile + lr][16 ks + 4 lg .. +3].  Rows of inactive
    // steps are zero (selected, so a NaN there cannot enter a product).
    u32x2 kf[4][kDk / 16], kw[kDk / 16], qf[kDk / 16];
    const size_t kq_row = static_cast<size_t>(Hk) * kDk * 2;   // bytes per step
    const size_t kq_base = (static_cast<size_t>(b) * T * Hk + hk) * kDk * 2;
#pragma unroll
    for (int tile = 0; tile < 4; ++tile) {
        const uint32_t t = t0 + 16u * tile + lr;
        const bool act = step_active(mask, b, T, t);
        const size_t off = kq_base + static_cast<size_t>(t < T ? t : 0) * kq_row + lg * 8;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) {
            const u32x2 kv = t < T ? load8(k, off + ks * 32) : zero2();
            kf[tile][ks] = act ? kv : zero2();
        }
    }
    {
        const uint32_t t = t0 + 16u * w + lr;
        const bool act = step_active(mask, b, T, t);
        const size_t off = kq_base + static_cast<size_t>(t < T ? t : 0) * kq_row + lg * 8;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) {
            const u32x2 kv = t < T ? load8(k, off + ks * 32) : zero2();
            const u32x2 qv = t < T ? load8(q, off + ks * 32) : zero2();
            kw[ks] = act ? kv : zero2();
            qf[ks] = act ? qv : zero2();
        }
    }
    __syncthreads();

    // M by running products of the gates: thread t walks s = t, t-1, .., 0.
    if (tid < kC) {
        const int t = static_cast<int>(tid);
        float p = 1.0f;
        for (int s = kC - 1; s >= 0; --s) {
            Ml[t * MS + s] = s <= t ? p : 0.0f;
            if (s <= t) p *= gs[s];
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
            Al[t * AS + s] = s < t ? bs[t] * (m * (G[r] + G2[r])) : 0.0f;
            uint16_t hi, lo;
            split1(s <= t ? m * (H[r] + H2[r]) : 0.0f, hi, lo);
            phi[t * kC + s] = hi;
            plo[t * kC + s] = lo;
        }
    }
    __syncthreads();

    // (I + A)^-1 by forward substitution, one column per lane of wave 0:
    // col[i] = [i == c] - sum_{j<i} A[i,j] col[j].  Then Tb = (I + A)^-1 diag(beta).
    if (w == 0) {
        float col[kC];
        forward_row<0, AS>(col, Al, static_cast<int>(l));
        const float bc = bs[l];
        uint16_t* thi = reinterpret_cast<uint16_t*>(wsb + PrefillWs::kTbHi);
        uint16_t* tlo = reinterpret_cast<uint16_t*>(wsb + PrefillWs::kTbLo);
#pragma unroll
        for (int i = 0; i < kC; ++i) {
            uint16_t hi, lo;
            split1(col[i] * bc, hi, lo);
            thi[i * kC + l] = hi;
            tlo[i * kC + l] = lo;
        }
    }
}

// ------------------------------------------------------------------ scan
//
// One workgroup of four waves per (b, hv, 16 consecutive value rows).  The
// state is held transposed in MFMA accumulators: wave w owns key columns
// 32w .. 32w+31 (two 16 x 16 tiles), lane l holding S[dv0 + l%16][16 tile +
// 4 (l/16) + r] -- the layout in which a tile is also the B operand of
// X = K S^T for the key step it covers.  Wave w computes the chunk's step
// tile w (steps 16w .. 16w+15) of X, Delta and Y.
struct ScanIn {
    u32x2 kf[kDk / 16], qf[kDk / 16];   // K, Q [16w + lr][16 ks + 4 lg ..]
    u32x2 th[4], tl[4], ph[4], pl[4];   // Tb and P [16w + lr][16 ks + 4 lg ..]
    f32x4v v, gam, rho;                 // at steps 16w + 4 lg + r, row lr
    float gC;                           // gamma_63
    uint32_t act;                       // bit r: step 16w + 4 lg + r is active
};

template <int IO>
__device__ __forceinline__ void scan_load(ScanIn& in, const void* q, const void* k, const void* v,
                                          const uint32_t* mask, const unsigned char* wsb,
                                          uint32_t b, uint32_t hv, uint32_t hk, uint32_t dv0,
                                          uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dv,
                                          uint32_t t0, uint32_t w, uint32_t lr, uint32_t lg) {
    {
        const uint32_t t = t0 + 16u * w + lr;
        const bool act = step_active(mask, b, T, t);
        const size_t off = ((static_cast<size_t>(b) * T + (t < T ? t : 0)) * Hk + hk) * kDk * 2 + lg * 8;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) {
            const u32x2 kv = t < T ? load8(k, off + ks * 32) : zero2();
            const u32x2 qv = t < T ? load8(q, off + ks * 32) : zero2();
            in.kf[ks] = act ? kv : zero2();
            in.qf[ks] = act ? qv : zero2();
        }
    }
    in.act = 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t t = t0 + 16u * w + 4u * lg + r;
        const bool act = step_active(mask, b, T, t);
        const float vv = t < T ? io_load1<IO>(v, ((static_cast<size_t>(b) * T + t) * Hv + hv) * Dv + dv0 + lr)
                               : 0.0f;
        in.v[r] = act ? vv : 0.0f;
        in.act |= act ? (1u << r) : 0u;
    }
    const size_t frag = ((16u * w + lr) * kC + 4u * lg) * 2;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        in.th[ks] = load8(wsb, PrefillWs::kTbHi + frag + ks * 32);
        in.tl[ks] = load8(wsb, PrefillWs::kTbLo + frag + ks * 32);
        in.ph[ks] = load8(wsb, PrefillWs::kPHi + frag + ks * 32);
        in.pl[ks] = load8(wsb, PrefillWs::kPLo + frag + ks * 32);
    }
    const float* gam = reinterpret_cast<const float*>(wsb + PrefillWs::kGamma);
    const float* rho = reinterpret_cast<const float*>(wsb + PrefillWs::kRho);
    const float4 g4 = *reinterpret_cast<const float4*>(gam + 16u * w + 4u * lg);
    const float4 r4 = *reinterpret_cast<const float4*>(rho + 16u * w + 4u * lg);
    in.gam = f32x4v{g4.x, g4.y, g4.z, g4.w};
    in.rho = f32x4v{r4.x, r4.y, r4.z, r4.w};
    in.gC = gam[kC - 1];
}

template <int IO>
__global__ __launch_bounds__(256, 1) void gdn_prefill_scan_kernel(
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
    __shared__ __align__(16) u32x4 dfr[4][64];         // Delta
    __shared__ __align__(16) u32x4 dtf[4][64];         // rho o Delta
    __shared__ __align__(16) uint16_t kt[2][kDk * KTS];   // K^T [dk][t], two chunks

    const uint32_t tid = threadIdx.x, l = tid & 63u, w = tid >> 6;
    const uint32_t lr = l & 15u, lg = l >> 4;
    const uint32_t slices = Dv / kRows;
    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const uint32_t n = blk / slices;                    // b * Hv + hv
    const uint32_t dv0 = (blk - n * slices) * kRows;
    const uint32_t b = n / Hv, hv = n - b * Hv;
    const uint32_t hk = tiled ? hv % Hk : hv / group;

    // This lane's two 16-byte state pieces: row dv0 + lr, columns 32w + 16u + 4lg.
    const size_t srow = (static_cast<size_t>(n) * Dv + dv0 + lr) * kDk + 32u * w + 4u * lg;
    f32x4v acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float4 s4 = *reinterpret_cast<const float4*>(state_in + srow + 16 * u);
        acc[u] = f32x4v{s4.x, s4.y, s4.z, s4.w};
    }

    const unsigned char* wsn = ws + static_cast<size_t>(n) * nchunks * PrefillWs::kBytes;
    ScanIn cur, nxt;
    scan_load<IO>(nxt, q, k, v, mask, wsn, b, hv, hk, dv0, T, Hk, Hv, Dv, 0u, w, lr, lg);

    for (uint32_t c = 0; c < nchunks; ++c) {
        cur = nxt;
        if (c + 1 < nchunks)
            scan_load<IO>(nxt, q, k, v, mask, wsn + (c + 1) * static_cast<size_t>(PrefillWs::kBytes),
                          b, hv, hk, dv0, T, Hk, Hv, Dv, (c + 1) * kC, w, lr, lg);
        const uint32_t t0 = c * kC;
        uint16_t* ktb = kt[c & 1u];

        // State tiles of this wave -> (hi, lo) fragments for every wave.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            u32x2 hi, lo;
            split4(acc[u], hi, lo);
            sfr[2 * w + u][l] = u32x4{hi.x, hi.y, lo.x, lo.y};
        }
        // This wave's 16 key rows, transposed into K^T [dk][t].
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) {
            const uint32_t dk = 16u * ks + 4u * lg, t = 16u * w + lr;
            ktb[(dk + 0) * KTS + t] = static_cast<uint16_t>(cur.kf[ks].x);
            ktb[(dk + 1) * KTS + t] = static_cast<uint16_t>(cur.kf[ks].x >> 16);
            ktb[(dk + 2) * KTS + t] = static_cast<uint16_t>(cur.kf[ks].y);
            ktb[(dk + 3) * KTS + t] = static_cast<uint16_t>(cur.kf[ks].y >> 16);
        }
        __syncthreads();

        // X_K = K S0^T and X_Q = Q S0^T for step tile w (hi and lo parts apart).
        f32x4v xk = {0.f, 0.f, 0.f, 0.f}, xq = xk, xk2 = xk, xq2 = xk;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks) {
            const u32x4 s = sfr[ks][l];
            const u32x2 sh = {s.x, s.y}, sl = {s.z, s.w};
            xk = mfma_bf16(cur.kf[ks], sh, xk);
            xq = mfma_bf16(cur.qf[ks], sh, xq);
            xk2 = mfma_bf16(cur.kf[ks], sl, xk2);
            xq2 = mfma_bf16(cur.qf[ks], sl, xq2);
        }
        f32x4v R;
#pragma unroll
        for (int r = 0; r < 4; ++r) R[r] = cur.v[r] - cur.gam[r] * (xk[r] + xk2[r]);
        {
            u32x2 hi, lo;
            split4(R, hi, lo);
            rfr[w][l] = u32x4{hi.x, hi.y, lo.x, lo.y};
        }
        __syncthreads();

        // Delta (step tile w) = Tb R.  Tb and P are zero above the diagonal, so
        // the tiles past w add exact zeros; every wave runs all four, which
        // costs nothing on the critical path (wave 3 needs all four anyway).
        f32x4v D = {0.f, 0.f, 0.f, 0.f}, D2 = D;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4 rr = rfr[ks][l];
            const u32x2 rh = {rr.x, rr.y}, rl = {rr.z, rr.w};
            D = mfma_bf16(cur.th[ks], rh, D);
            D2 = mfma_bf16(cur.th[ks], rl, D2);
            D2 = mfma_bf16(cur.tl[ks], rh, D2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) D[r] += D2[r];
        {
            u32x2 hi, lo;
            split4(D, hi, lo);
            dfr[w][l] = u32x4{hi.x, hi.y, lo.x, lo.y};
            f32x4v Dt;
#pragma unroll
            for (int r = 0; r < 4; ++r) Dt[r] = cur.rho[r] * D[r];
            split4(Dt, hi, lo);
            dtf[w][l] = u32x4{hi.x, hi.y, lo.x, lo.y};
        }
        if (delta_log) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (cur.act & (1u << r)) {
                    const size_t i = ((static_cast<size_t>(b) * T + t0 + 16u * w + 4u * lg + r) * Hv + hv) * Dv +
                                     dv0 + lr;
                    static_cast<uint16_t*>(delta_log)[i] = static_cast<uint16_t>(f32_to_bf16_bits(D[r]));
                }
            }
        }
        __syncthreads();

        // Y (step tile w) = gamma o X_Q + P Delta.
        f32x4v Y, Y2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) Y[r] = cur.gam[r] * (xq[r] + xq2[r]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4 dd = dfr[ks][l];
            const u32x2 dh = {dd.x, dd.y}, dl = {dd.z, dd.w};
            Y = mfma_bf16(cur.ph[ks], dh, Y);
            Y2 = mfma_bf16(cur.ph[ks], dl, Y2);
            Y2 = mfma_bf16(cur.pl[ks], dh, Y2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (cur.act & (1u << r)) {
                const size_t i = ((static_cast<size_t>(b) * T + t0 + 16u * w + 4u * lg + r) * Hv + hv) * Dv + dv0 + lr;
                static_cast<uint16_t*>(y)[i] = static_cast<uint16_t>(f32_to_bf16_bits(Y[r] + Y2[r]));
            }
        }

        // S^T <- gamma_63 S^T + K^T (rho o Delta) for this wave's key tiles.
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[u][r] *= cur.gC;
        f32x4v lo_acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4 dd = dtf[ks][l];
            const u32x2 dh = {dd.x, dd.y}, dl = {dd.z, dd.w};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t dk = 16u * (2u * w + u) + lr;
                const u32x2 a = *reinterpret_cast<const u32x2*>(&ktb[dk * KTS + 16 * ks + 4 * lg]);
                acc[u] = mfma_bf16(a, dh, acc[u]);
                lo_acc[u] = mfma_bf16(a, dl, lo_acc[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[u][r] += lo_acc[u][r];
    }

#pragma unroll
    for (int u = 0; u < 2; ++u)
        *reinterpret_cast<float4*>(state_out + srow + 16 * u) = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
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
    hipLaunchKernelGGL(gdn_prefill_scan_kernel<kBF16>, dim3(a.B * a.Hv * (a.Dv / kRows)), dim3(256), 0, stream,
                       a.q, a.k, a.v, a.state_in, a.mask, ws, a.y, a.state_out, a.delta_log, a.T, a.Hk, a.Hv,
                       a.Dv, nchunks, group, tiled);
    return hipGetLastError();
}

}  // namespace gdn
