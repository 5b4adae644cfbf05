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
// (scan) carries the state through the chunks in order, with every product on
// the 16 x 16 x 32 bf16 matrix instruction: X = [K; Q] S0^T, Delta = Tb R,
// Y = gamma o XQ + P Delta and S^T <- gamma_63 S^T + K^T (rho o Delta),
// rho_s = M[63,s].  Key widths 128 and 192 (the 192-wide key heads of the
// record page's shape-cell instances), bf16 or fp16 I/O.
//
// Precision.  bf16 keys and queries enter the MFMAs exactly.  An fp16 key or
// query element (11 significant bits) is split exactly into two bf16 numbers
// hi = round(x), lo = x - hi.  Every fp32 operand (the state, R, Delta, Tb, P)
// enters as hi + lo, two bf16 numbers with hi = round(x) and lo = round(x - hi)
// (about 16 significant bits).  A product of two split operands takes three
// MFMAs (hi.hi + hi.lo + lo.hi), a bf16 x split product two; the Gram
// matrices of fp16 keys and queries take all four.  Accumulation is fp32.  M
// is formed by products of the gates (no division), so zero or tiny gates are
// exact.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

#include <atomic>

namespace gdn {
namespace {

constexpr int kC = 64;            // steps per chunk
constexpr int kRows = 16;         // state rows per scan workgroup

typedef float f32x4v __attribute__((ext_vector_type(4)));

// D += A B on gfx950's double-depth bf16 tile: 16 x 16 x 32, eight bf16 of
// A (row l % 16) and of B (column l % 16) per lane, over the same eight
// positions of the 32-deep sum in both, so that any operands whose lanes
// pair the same summation index give the full product.  D comes back as
// D[4 (l / 16) + r][l % 16], r = 0..3.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4v mfma_bf16_k32(u32x4 a, u32x4 b, f32x4v acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                   0, 0, 0);
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

// An input element's bits as fp32.
template <int IO>
__device__ __forceinline__ float in_f32(uint32_t bits) {
    return IO == kBF16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
}

// Eight fp16 values (one 16-byte piece, element order kept) as two bf16
// pieces with hi + lo equal to each value exactly: rounding an 11-bit
// significand to bf16's 8 bits leaves a remainder of at most 4 significant
// bits, inside bf16's exponent range for every finite fp16 number.
__device__ __forceinline__ void split_f16x8(const u32x4& raw, u32x4& hi, u32x4& lo) {
    uint32_t h[4], o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = f16_bits_to_f32(raw[i] & 0xffffu), b = f16_bits_to_f32(raw[i] >> 16);
        h[i] = cvt_pk_bf16(a, b);
        o[i] = cvt_pk_bf16(a - __uint_as_float(h[i] << 16), b - __uint_as_float(h[i] & 0xffff0000u));
    }
    hi = u32x4{h[0], h[1], h[2], h[3]};
    lo = u32x4{o[0], o[1], o[2], o[3]};
}
__device__ __forceinline__ void split_f16x4(const u32x2& raw, u32x2& hi, u32x2& lo) {
    const u32x4 r4 = {raw.x, raw.y, 0u, 0u};
    u32x4 h4, l4;
    split_f16x8(r4, h4, l4);
    hi = u32x2{h4.x, h4.y};
    lo = u32x2{l4.x, l4.y};
}

__device__ __forceinline__ void split1(float x, uint16_t& hi, uint16_t& lo) {
    const uint32_t h = cvt_pk_bf16(x, 0.0f) & 0xffffu;
    hi = static_cast<uint16_t>(h);
    lo = static_cast<uint16_t>(cvt_pk_bf16(x - bf16_bits_to_f32(h), 0.0f));
}

}  // namespace

// Per (b, hv, chunk) block of the workspace, written by prep and read by scan.
// Tb and P are stored in the A-operand order of the 16 x 16 x 32 matrix
// instruction: block (tt * 2 + kb) of 2 KiB holds, for lane l = 16 lg + lr,
// the hi bf16 parts of M[16 tt + lr][32 kb + 8 lg .. +7] in its 16-byte slot
// l and the lo parts in slot 64 + l, so a wave reads one step tile's operands
// with fully coalesced 1 KiB loads (whole cache lines).  Both matrices are
// zero above the diagonal: blocks kb = 1 of step tiles 0 and 1 are never read.
struct PrefillWs {
    static constexpr int kMat = kC * kC * 2;             // one 64 x 64 bf16 matrix
    static constexpr int kTb = 0, kP = 2 * kMat;         // Tb, P: hi/lo fragment slots, 16 KiB each
    static constexpr int kGamma = 4 * kMat;              // gamma_t, fp32 [64]
    static constexpr int kRho = kGamma + kC * 4;         // rho_t = M[63, t], fp32 [64]
    static constexpr int kBytes = kRho + kC * 4;         // 33280
};

namespace {

// Byte offset of element [t][s] of a 64 x 64 matrix in the fragment order of
// PrefillWs (its hi part; the lo part is kFragLo bytes further).
constexpr uint32_t kFragLo = 1024;
__device__ __forceinline__ uint32_t frag_offset(uint32_t t, uint32_t s) {
    return ((t >> 4) * 2u + (s >> 5)) * 2048u + (16u * ((s & 31u) >> 3) + (t & 15u)) * 16u + (s & 7u) * 2u;
}

// Row I of the forward substitution (I + A) T = identity, then the rows after
// it, column by column, right-looking.  Four consecutive lanes share column c
// of T; lane q of the four owns rows i = 4m + q: it keeps their running sums
// sum[m] = sum_{j < I} A[i, j] T[j, c] and, once row i is reached, T[i, c] in
// mine[m].  Row I's owner forms T[I, c] = [I == c] - sum, a quad broadcast
// hands it to the other three lanes, and every lane adds A[i, I] T[I, c] to
// the sums of its rows.  A is read from LDS in the quad layout (aq_index):
// the 16 floats A[4m + q, j], m = 0..15, of column j and quad lane q form one
// 64-byte row, whose four 16-byte groups m/4 = 0..3 are stored at group
// m/4 ^ (q/2) ^ (j % 4): the four addresses the lanes of a quad read at once
// (the same for every column) fall on different banks, and so do most of the
// writes of a wave.  One 16-byte read covers four of a lane's rows.  The lane
// passes base pointers pe and po for stored groups of even and odd order, so
// every read address is a constant offset from one of them.  A is
// stored with zeros at and above the diagonal, so the sums of rows at or
// before I (already used) are the only ones that receive zero terms.  Row
// indices are template parameters so that the sums stay in registers; the
// dependency from one row to the next is a subtraction, the broadcast and one
// multiply-add.
__device__ __forceinline__ uint32_t aq_index(uint32_t i, uint32_t j) {      // float index of A[i, j]
    const uint32_t q = i & 3u, m = i >> 2;
    return (j * 4u + q) * 16u + ((((m >> 2) ^ (q >> 1) ^ j) & 3u) << 2) + (m & 3u);
}

// Row I's reads of A: the groups m4 >= I / 16 of column I (group m4 holds A at
// the lane's four rows among 16 m4 .. 16 m4 + 15; earlier groups' rows are all
// at or before I and take no more terms).
template <int I>
__device__ __forceinline__ void load_a_row(float4 (&a)[4], const float* pe, const float* po) {
#pragma unroll
    for (int m4 = (I >> 2) / 4; m4 < 4; ++m4) {
        const int v = m4 ^ (I & 3);                                 // stored group, before the lane's q/2
        a[m4] = *reinterpret_cast<const float4*>((v & 1 ? po : pe) + I * 64 + 4 * v);
    }
}

// cur holds row I's reads of A; row I + 1's are issued before row I's work,
// so they are on their way during it.
template <int I>
__device__ __forceinline__ void forward_right_row(float (&sum)[16], float (&mine)[16], const float* pe,
                                                  const float* po, int c, int q, const float4 (&cur)[4]) {
    constexpr int M0 = I >> 2, Q0 = I & 3;
    float4 nxt[4];
    if constexpr (I + 1 < kC) load_a_row<I + 1>(nxt, pe, po);
    const float own = (I == c ? 1.0f : 0.0f) - sum[M0];            // meaningful on lane Q0 of the quad
    const float tI = dpp_read<Q0 * 0x55>(own);                      // quad_perm [Q0, Q0, Q0, Q0]
    mine[M0] = q == Q0 ? tI : mine[M0];
#pragma unroll
    for (int m4 = M0 / 4; m4 < 4; ++m4) {
        const float4 a = cur[m4];
        if (4 * m4 + 0 >= M0) sum[4 * m4 + 0] = fmaf(a.x, tI, sum[4 * m4 + 0]);
        if (4 * m4 + 1 >= M0) sum[4 * m4 + 1] = fmaf(a.y, tI, sum[4 * m4 + 1]);
        if (4 * m4 + 2 >= M0) sum[4 * m4 + 2] = fmaf(a.z, tI, sum[4 * m4 + 2]);
        if (4 * m4 + 3 >= M0) sum[4 * m4 + 3] = fmaf(a.w, tI, sum[4 * m4 + 3]);
    }
    if constexpr (I + 1 < kC) forward_right_row<I + 1>(sum, mine, pe, po, c, q, nxt);
}

// The substitution from row I0 on.
template <int I0>
__device__ __forceinline__ void forward_right_from(float (&sum)[16], float (&mine)[16], const float* pe,
                                                   const float* po, int c, int q) {
    float4 first[4];
    load_a_row<I0>(first, pe, po);
    forward_right_row<I0>(sum, mine, pe, po, c, q, first);
}

// ------------------------------------------------------------------ prep
//
// One workgroup of four waves per (b, key head, chunk) and up to kPrepHeads
// of the value heads that read that key head.  The Gram products G = K K^T
// and H = Q K^T of a chunk depend on the key head only, so they are formed
// once from one load of the key and query rows; the gates and betas, M, A,
// P, (I + A)^-1 and Tb are then taken value head by value head.  Wave w owns
// row tile w (steps 16w .. 16w+15) of the 64 x 64 matrices.
//
// LDS of the prep kernel (36 KiB at Dk = 128: four workgroups per CU; 44 KiB
// at Dk = 192: three).  Only the chunk's key rows (padded rows) are staged:
// each wave loads the 16 query rows of its own row tile straight into the
// registers of its Gram product.  P (in the workspace's fragment order)
// takes the key rows' space once the Gram tiles are formed.  M, then A (in
// the quad layout), then Tb (fragment order) share one area: A is held in
// registers until every wave is done reading M, and Tb until every wave is
// done reading A.  A value head's Tb and P leave for the workspace before
// the next value head's M and P take their places.
constexpr uint32_t kPrepHeads = 4;     // value heads per prep workgroup, at most

template <int DK>
struct PrepLds {
    static constexpr int KS = DK * 2 + 16;             // K row stride in bytes (padded)
    static constexpr int MS = kC + 1;                  // M row stride in floats
    static constexpr int KR = 0;                       // K rows [64] x KS
    static constexpr int PO = KR;                      // then P, hi and lo fragments (16 KiB)
    static constexpr int ML = KR + kC * KS;            // M [64][65] fp32
    static constexpr int AQ = ML;                      // then A in the quad layout (16 KiB)
    static constexpr int TBO = ML;                     // then Tb, hi and lo fragments (16 KiB)
    static constexpr int GS = ML + kC * MS * 4;        // gates [kPrepHeads][64] fp32
    static constexpr int BS = GS + kPrepHeads * kC * 4;   // betas [kPrepHeads][64] fp32
    static constexpr int BYTES = BS + kPrepHeads * kC * 4;
    static_assert(PrefillWs::kP - PrefillWs::kTb == 2 * PrefillWs::kMat, "Tb then P in the workspace");
    static_assert(2 * PrefillWs::kMat <= kC * KS, "P fits where the key rows were");
    static_assert(kC * 4 * 16 * 4 <= kC * MS * 4, "A fits where M was");
    static_assert(2 * PrefillWs::kMat <= kC * MS * 4, "Tb fits where A was");
};

template <int IO, int DK>
__global__ __launch_bounds__(256, 2) void gdn_prefill_prep_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ g,
    const void* __restrict__ beta, const uint32_t* __restrict__ mask,
    unsigned char* __restrict__ ws, void* __restrict__ k_log, void* __restrict__ g_log,
    uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t nchunks, uint32_t group, uint32_t head_sets, int tiled)
{
    static_assert(IO == kBF16 || IO == kF16, "the chunked prefill takes 16-bit I/O");
    using PrepLds = gdn::PrepLds<DK>;
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int MS = PrepLds::MS;
    float* gs = reinterpret_cast<float*>(lds + PrepLds::GS);
    float* bs = reinterpret_cast<float*>(lds + PrepLds::BS);
    float* Ml = reinterpret_cast<float*>(lds + PrepLds::ML);
    float* Aq = reinterpret_cast<float*>(lds + PrepLds::AQ);

    const uint32_t tid = threadIdx.x, l = tid & 63u, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t lr = l & 15u, lg = l >> 4;
    // Workgroup order: (b, chunk, key head, set of value heads), the last
    // fastest, so that the workgroups of one XCD read whole steps' rows of
    // every key head (contiguous memory).  Set hs takes the value heads
    // j = kPrepHeads hs .. of the key head (j-th value head: hk + Hk j under
    // the tiled map, hk group + j under the block map).
    uint32_t li = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const uint32_t hs = li % head_sets;
    li /= head_sets;
    const uint32_t hk = li % Hk;
    li /= Hk;
    const uint32_t c = li % nchunks, b = li / nchunks;
    const uint32_t j0 = hs * kPrepHeads;
    const uint32_t nh = group - j0 < kPrepHeads ? group - j0 : kPrepHeads;   // value heads here
    auto value_head = [&](uint32_t jj) { return tiled ? hk + Hk * (j0 + jj) : hk * group + j0 + jj; };
    const uint32_t t0 = c * kC;

    // The chunk's key rows, 16-byte pieces: thread tid takes pieces
    // p = tid + 256 j, piece p % (DK / 8) of row p / (DK / 8).  The query rows
    // of this wave's row tile: lane (lr, lg) takes row 16 w + lr, pieces
    // 4 m + lg (its A operand of the Gram product below).  Thread tid also
    // takes the gate and beta of step tid % 64 of value head tid / 64.  Steps
    // past T read step T-1; rows of inactive steps become zeros (a select, so
    // a NaN there cannot enter a product).
    // Mask words are loaded whether or not there is a mask (from k, whose
    // B*T*Hk*Dk/2 words cover every index, when there is none) and then
    // selected, so the loads are not serialised behind branches.
    constexpr uint32_t kPieces = DK / 8;               // 16-byte pieces per row
    constexpr int kPer = kC * kPieces / 256;           // pieces per thread
    constexpr int NB = DK / 32;                        // 32-column key blocks
    static_assert(kPrepHeads * kC == 256, "one gate per thread");
    const uint32_t* mwords = mask ? mask : static_cast<const uint32_t*>(k);
    u32x4 qf[NB];                                      // query pieces of row 16 w + lr
    {
        const uint32_t t = t0 + 16u * w + lr, tc = t < T ? t : T - 1;
        const size_t off = ((static_cast<size_t>(b) * T + tc) * Hk + hk) * (DK * 2) + lg * 16;
#pragma unroll
        for (int m = 0; m < NB; ++m)
            qf[m] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(q) + off + m * 64);
        const uint32_t mword = mwords[static_cast<size_t>(b) * T + tc];
        const bool act = t < T && (mask ? mword : 1u) > 0u;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int m = 0; m < NB; ++m) qf[m] = act ? qf[m] : z;
    }
    {
        u32x4 kp[kPer];
        uint32_t mw[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t p = tid + 256u * j, row = p / kPieces, pc = p - row * kPieces;
            const uint32_t t = t0 + row, tc = t < T ? t : T - 1;
            const size_t off = ((static_cast<size_t>(b) * T + tc) * Hk + hk) * (DK * 2) + pc * 16;
            kp[j] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(k) + off);
            const uint32_t m = mwords[static_cast<size_t>(b) * T + tc];
            mw[j] = mask ? m : 1u;
        }
        {
            const uint32_t jj = tid / kC, ts = tid % kC;
            const uint32_t jc = jj < nh ? jj : 0u;         // heads past nh load head 0's (unused)
            const uint32_t hv = value_head(jc);
            const uint32_t t = t0 + ts, tc = t < T ? t : T - 1;
            const size_t i = (static_cast<size_t>(b) * T + tc) * Hv + hv;
            const uint32_t graw = static_cast<const uint16_t*>(g)[i];
            const float bl = io_load1<IO>(beta, i);
            const uint32_t mword = mwords[static_cast<size_t>(b) * T + tc];
            const bool act = t < T && (mask ? mword : 1u) > 0u;
            gs[tid] = act ? in_f32<IO>(graw) : 1.0f;
            bs[tid] = act ? bl : 0.0f;
            if (g_log != nullptr && act && jj < nh)               // tape capture: the gate's bits
                static_cast<uint16_t*>(g_log)[(static_cast<size_t>(b) * T + t) * Hv + hv] =
                    static_cast<uint16_t>(graw);
        }
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t p = tid + 256u * j, r = p / kPieces, pc = p - r * kPieces;
            const bool act = t0 + r < T && mw[j] > 0u;
            *reinterpret_cast<u32x4*>(lds + PrepLds::KR + r * PrepLds::KS + pc * 16) = act ? kp[j] : z;
            if (k_log != nullptr && act)                         // tape capture: the key row of each value head
                for (uint32_t jj = 0; jj < nh; ++jj)
                    *reinterpret_cast<u32x4*>(static_cast<char*>(k_log) +
                                              ((static_cast<size_t>(b) * T + t0 + r) * Hv + value_head(jj)) *
                                                  (DK * 2) +
                                              pc * 16) = kp[j];
        }
    }
    __syncthreads();

    // Gram tiles G = K K^T and H = Q K^T of row tile w (all four column tiles;
    // above the diagonal the s <= t masks below make A and P exact zeros).
    // Products of bf16 values are exact in fp32 (fp16 inputs: of their hi and
    // lo parts).  32-deep products over key columns: lane holds
    // x[16 tile + lr][32 m + 8 lg .. +7] as A and B.
    f32x4v G[4], H[4];
    {
        u32x4 kw[NB], kwl[NB], qfl[NB];
        const unsigned char* kwr = lds + PrepLds::KR + (16u * w + lr) * PrepLds::KS + lg * 16;
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            kw[m] = *reinterpret_cast<const u32x4*>(kwr + m * 64);
            if constexpr (IO == kF16) {
                split_f16x8(kw[m], kw[m], kwl[m]);
                split_f16x8(qf[m], qf[m], qfl[m]);
            }
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const unsigned char* kr = lds + PrepLds::KR + (16u * st + lr) * PrepLds::KS + lg * 16;
            f32x4v gg = {0.f, 0.f, 0.f, 0.f}, hh = gg;
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                u32x4 bk = *reinterpret_cast<const u32x4*>(kr + m * 64);
                if constexpr (IO == kBF16) {
                    gg = mfma_bf16_k32(kw[m], bk, gg);
                    hh = mfma_bf16_k32(qf[m], bk, hh);
                } else {
                    u32x4 bkl;
                    split_f16x8(bk, bk, bkl);
                    gg = mfma_bf16_k32(kw[m], bk, gg);
                    gg = mfma_bf16_k32(kw[m], bkl, gg);
                    gg = mfma_bf16_k32(kwl[m], bk, gg);
                    gg = mfma_bf16_k32(kwl[m], bkl, gg);
                    hh = mfma_bf16_k32(qf[m], bk, hh);
                    hh = mfma_bf16_k32(qf[m], bkl, hh);
                    hh = mfma_bf16_k32(qfl[m], bk, hh);
                    hh = mfma_bf16_k32(qfl[m], bkl, hh);
                }
            }
            G[st] = gg;
            H[st] = hh;
        }
    }
    __syncthreads();       // the key rows are dead

    for (uint32_t jj = 0; jj < nh; ++jj) {
        // tid, l, lr and lg shadow the kernel's own on purpose: the thread
        // index passes through an empty asm statement so that the addresses
        // derived from it are formed per value head, not kept in registers
        // across the loop (which pushed the kernel to 196 VGPRs).
        uint32_t tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const uint32_t l = tid & 63u, lr = l & 15u, lg = l >> 4;
        const uint32_t hv = value_head(jj);
        const uint32_t n = b * Hv + hv;
        unsigned char* wsb = ws + (static_cast<size_t>(n) * nchunks + c) * PrefillWs::kBytes;
        const float* gh = gs + jj * kC;
        const float* bh = bs + jj * kC;

        // M[t, s] = g_{s+1} .. g_t (s <= t) by products of the gates, no
        // division, over all four waves: thread (t = tid / 4, q = tid % 4) takes
        // columns 16 q .. 16 q + 15 of row t.  It forms the product of its
        // segment's gates up to t, the quad (the four segments of row t) hands
        // it the product of the later segments' ones, and it walks its columns
        // down from there, multiplying in g_s once s <= t.
        {
            const int t = static_cast<int>(tid >> 2), q = static_cast<int>(tid & 3u);
            float gq[16];
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const float4 v4 = *reinterpret_cast<const float4*>(&gh[16 * q + 4 * i4]);
                gq[4 * i4] = v4.x; gq[4 * i4 + 1] = v4.y; gq[4 * i4 + 2] = v4.z; gq[4 * i4 + 3] = v4.w;
            }
            float seg = 1.0f;                                           // g over this segment, up to t
#pragma unroll
            for (int i = 15; i >= 0; --i) seg = 16 * q + i <= t ? seg * gq[i] : seg;
            // (The reads run on every lane of the quad, then are selected: a
            // read from a lane that is switched off would return 0.)
            const float d1 = dpp_read<0xf9>(seg);                       // quad_perm [1,2,3,3]: segment q + 1
            const float d2 = dpp_read<0xfe>(seg);                       // quad_perm [2,3,3,3]: segment q + 2
            const float d3 = dpp_read<0xff>(seg);                       // quad_perm [3,3,3,3]: segment q + 3
            float r = (q < 3 ? d1 : 1.0f) * (q < 2 ? d2 : 1.0f) * (q < 1 ? d3 : 1.0f);   // later segments, up to t
            if (q == 0) reinterpret_cast<float*>(wsb + PrefillWs::kGamma)[t] = seg * r;   // gamma_t = g_0 .. g_t
#pragma unroll
            for (int i = 15; i >= 0; --i) {
                const int sc = 16 * q + i;
                Ml[t * MS + sc] = sc <= t ? r : 0.0f;
                r = sc <= t ? r * gq[i] : r;
            }
        }
        __syncthreads();   // M is complete

        // A and P of row tile w; P goes to its LDS area, A stays in registers
        // until M is dead.
        if (tid < kC) reinterpret_cast<float*>(wsb + PrefillWs::kRho)[tid] = Ml[(kC - 1) * MS + tid];
        unsigned char* op = lds + PrepLds::PO;
        f32x4v A[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * static_cast<int>(w) + 4 * static_cast<int>(lg) + r;
                const int s = 16 * st + static_cast<int>(lr);
                const float m = Ml[t * MS + s];
                A[st][r] = s < t ? bh[t] * (m * G[st][r]) : 0.0f;
                uint16_t hi, lo;
                split1(s <= t ? m * H[st][r] : 0.0f, hi, lo);
                const uint32_t o = frag_offset(static_cast<uint32_t>(t), static_cast<uint32_t>(s));
                *reinterpret_cast<uint16_t*>(op + o) = hi;
                *reinterpret_cast<uint16_t*>(op + o + kFragLo) = lo;
            }
        }
        __syncthreads();   // M is dead
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Aq[aq_index(16u * w + 4u * lg + r, 16u * st + lr)] = A[st][r];
        }
        __syncthreads();

        // (I + A)^-1 by forward substitution over all four waves (four lanes per
        // column), then Tb = (I + A)^-1 diag(beta).
        {
            const int col = static_cast<int>(tid >> 2), qq = static_cast<int>(tid & 3u);
            float mine[16], sum[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) mine[m] = sum[m] = 0.0f;
            const int x = qq >> 1;                                       // group order m/4 ^ x
            const float* pe = Aq + qq * 16 + 4 * x;
            const float* po = Aq + qq * 16 - 4 * x;
            // Wave w holds columns 16w .. 16w+15, and T[i, c] = 0 exactly for
            // i < c: its rows before 16w add exact zeros and are skipped.
            switch (w) {
                case 0: forward_right_from<0>(sum, mine, pe, po, col, qq); break;
                case 1: forward_right_from<16>(sum, mine, pe, po, col, qq); break;
                case 2: forward_right_from<32>(sum, mine, pe, po, col, qq); break;
                default: forward_right_from<48>(sum, mine, pe, po, col, qq); break;
            }
            const float bc = bh[col];
            __syncthreads();                                             // every wave is done reading A
            unsigned char* otb = lds + PrepLds::TBO;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int i = 4 * m + qq;
                uint16_t hi, lo;
                split1(mine[m] * bc, hi, lo);
                const uint32_t o = frag_offset(static_cast<uint32_t>(i), static_cast<uint32_t>(col));
                *reinterpret_cast<uint16_t*>(otb + o) = hi;
                *reinterpret_cast<uint16_t*>(otb + o + kFragLo) = lo;
            }
        }
        __syncthreads();

        // The 32 KiB of Tb and P (already in fragment order) to the workspace in
        // contiguous 16-byte pieces.
        constexpr int kOutPer = 2 * PrefillWs::kMat / 16 / 256;          // pieces per thread of each matrix
#pragma unroll
        for (int j = 0; j < kOutPer; ++j) {
            const uint32_t p = tid + 256u * j;
            *reinterpret_cast<u32x4*>(wsb + PrefillWs::kTb + p * 16) =
                *reinterpret_cast<const u32x4*>(lds + PrepLds::TBO + p * 16);
            *reinterpret_cast<u32x4*>(wsb + PrefillWs::kP + p * 16) =
                *reinterpret_cast<const u32x4*>(lds + PrepLds::PO + p * 16);
        }
        if (jj + 1 < nh) __syncthreads();   // the next value head's M and P take these areas
    }
}

// ------------------------------------------------------------------ scan
//
// One workgroup of eight waves per (b, hv, 16 consecutive value rows).  The
// state is held transposed in MFMA accumulators: wave w owns the sixteen key
// columns kcol(w, 0..15) (key tile w), lane l holding
// S[dv0 + l%16][kcol(w, 4 (l/16) + r)]; with 192 key columns waves 4-7 also
// own key tiles 8-11 (tile w + 4).  The hi and lo parts of tiles 2m and 2m+1
// side by side are the B operand of the 32-deep product X = K S^T over key
// columns 32m .. 32m + 31.
// Waves 0-3 (the K side) take step tile w of the chunk: X_K, R and Delta.
// Waves 4-7 (the Q side) take step tile w-4: X_Q, and Y of the previous chunk
// while the K side solves for Delta (Y is not on the state's dependency chain).
//
// Each lane loads its key or query pieces straight from the input two chunks
// ahead: with the key index permuted (kcol), the eight key columns a lane
// multiplies are one contiguous 16-byte piece of a row.  v of this row block,
// gamma, rho and the step flags come into registers two chunks ahead too and
// into LDS at the top of their chunk.  Tb and P are already in operand order
// in the workspace and go straight to registers, two chunks ahead.  Key,
// query and value rows of inactive steps (masked, or past T) are replaced by
// zeros.
template <int IO, int DK>
struct ScanLds {
    static constexpr int NB = DK / 32;                 // 32-column key blocks
    // Key rows in LDS: stride 2 DK + 64 bytes (an odd multiple of 64 bytes
    // modulo 256), and in rows t with t / 8 odd the two 8-byte halves of each
    // 16-byte piece swapped, so that the transposing reads of half a wave
    // (four rows of each of two 8-row groups) fall on distinct banks.
    static constexpr int KRS = DK * 2 + 64;
    static_assert(KRS % 256 == 64 || KRS % 256 == 192, "key row stride");
    static constexpr int SFR = 0;                      // state fragments [2 NB][64] x 16 B (hi [NB], lo [NB])
    static constexpr int BOP = 4 * 64 * 16;            // one step-indexed B operand (see bop_store)
    static constexpr int RFR = SFR + 2 * NB * 64 * 16; // R
    static constexpr int DFR = RFR + BOP;              // Delta, two chunks
    static constexpr int DTF = DFR + 2 * BOP;          // rho o Delta
    static constexpr int KT = DTF + 4 * 64 * 16;       // K [t][dk] bf16, natural key order (fp16 keys: the hi part)
    static constexpr int KTL = KT + kC * KRS;          // the lo part of K (fp16 keys)
    static constexpr int VR = KTL + (IO == kF16 ? kC * KRS : 0);   // v rows [64] x 32 B (this row block)
    static constexpr int GR = VR + kC * 32;            // gamma [64], rho [64] fp32
    static constexpr int AF = GR + 2 * kC * 4;         // active flags [64] u32 (0 or 1)
    static constexpr int OT = AF + kC * 4;             // per wave: its pending output tile [16][16] bf16
    static constexpr int OTF = OT + 8 * 16 * 16 * 2;   // per wave: that tile's row flags [16] u32
    static constexpr int BYTES = OTF + 8 * 16 * 4;
};

// Staging registers: this thread's pieces of the next chunk.
struct ScanStage {
    u32x4 gv;             // threads 0-31: gamma/rho piece; threads 32-159: v piece
    uint32_t mv;          // threads 32-223: mask word of the v row / flag row (any word without a mask)
};

template <class L>
__device__ __forceinline__ void stage_store(const ScanStage& st, bool has_mask, unsigned char* lds, uint32_t T,
                                            uint32_t t0,
                                            uint32_t tid) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (tid < 32u) {
        *reinterpret_cast<u32x4*>(lds + L::GR + tid * 16) = st.gv;
    } else if (tid < 160u) {
        const uint32_t p = tid - 32u, vr = p >> 1;
        const bool act = t0 + vr < T && (!has_mask || st.mv > 0u);
        *reinterpret_cast<u32x4*>(lds + L::VR + vr * 32 + (p & 1u) * 16) = act ? st.gv : z;
    } else if (tid < 224u) {
        const uint32_t r = tid - 160u;
        reinterpret_cast<uint32_t*>(lds + L::AF)[r] = t0 + r < T && (!has_mask || st.mv > 0u) ? 1u : 0u;
    }
}

__device__ __forceinline__ u32x2 lo2(const u32x4& x) { return u32x2{x.x, x.y}; }
__device__ __forceinline__ u32x2 hi2(const u32x4& x) { return u32x2{x.z, x.w}; }

// Key column of index i (0..15) of key step ks: the key steps are a
// permutation of the key columns in which steps 2m and 2m+1 take, for each
// group g of four indices, the eight consecutive columns 32m + 8g .. 32m + 8g + 7
// (step 2m the first four, 2m+1 the last four).  Each lane's fragments of two
// key steps are then one contiguous 16-byte piece of a key row, and each
// lane's state piece stays contiguous too.  The contractions run over all
// key columns either way.
__device__ __forceinline__ uint32_t kcol(uint32_t ks, uint32_t i) {
    return 32u * (ks >> 1) + 8u * (i >> 2) + 4u * (ks & 1u) + (i & 3u);
}

// Four bf16 values by gfx950's transposing LDS read (ds_read_b64_tr_b16):
// within each group of 16 lanes, lane j receives element j % 4 of the 8-byte
// pieces that lanes j / 4 + 4 k (k = 0..3) address, in that order of k.
typedef short i16x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* p) {
    typedef __attribute__((address_space(3))) i16x4v lds_i16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

// A [64 steps][16 columns] operand split into hi and lo bf16 parts, written
// by the wave that holds step tile tt as an accumulator (lane 16 lg + lr:
// rows 16 tt + 4 lg .. +3 of column lr) and read as the B operand of 32-deep
// products over steps: hi of block kb at 16-byte slot kb * 64 + l, lo 2 KiB
// further, lane 16 lg' + lr holding rows 32 kb + 8 lg' .. +7 of column lr.
__device__ __forceinline__ void bop_store(unsigned char* base, uint32_t tt, uint32_t lr, uint32_t lg, u32x2 hi,
                                          u32x2 lo) {
    const uint32_t o = ((tt >> 1) * 64u + 16u * (2u * (tt & 1u) + (lg >> 1)) + lr) * 16u + (lg & 1u) * 8u;
    *reinterpret_cast<u32x2*>(base + o) = hi;
    *reinterpret_cast<u32x2*>(base + 2048 + o) = lo;
}
__device__ __forceinline__ u32x4 bop_hi(const unsigned char* base, uint32_t kb, uint32_t l) {
    return *reinterpret_cast<const u32x4*>(base + (kb * 64u + l) * 16u);
}
__device__ __forceinline__ u32x4 bop_lo(const unsigned char* base, uint32_t kb, uint32_t l) {
    return *reinterpret_cast<const u32x4*>(base + 2048 + (kb * 64u + l) * 16u);
}

template <int IO, int DK>
__global__ __launch_bounds__(512, 1) void gdn_prefill_scan_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* state_in, const uint32_t* __restrict__ mask,
    const unsigned char* __restrict__ ws, void* __restrict__ y, float* state_out,
    void* __restrict__ delta_log, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dv,
    uint32_t nchunks, uint32_t group, int tiled)
{
    static_assert(IO == kBF16 || IO == kF16, "the chunked prefill takes 16-bit I/O");
    static_assert(DK == 128 || DK == 192, "key width 128 or 192");
    using ScanLds = gdn::ScanLds<IO, DK>;
    constexpr int NB = DK / 32;
    extern __shared__ __align__(16) unsigned char lds[];
    u32x4 (*sfr)[64] = reinterpret_cast<u32x4 (*)[64]>(lds + ScanLds::SFR);
    unsigned char* const rfr = lds + ScanLds::RFR;
    unsigned char* const dfr = lds + ScanLds::DFR;      // chunk c at dfr + (c & 1) * BOP
    unsigned char* const dtf = lds + ScanLds::DTF;
    unsigned char* const ktb = lds + ScanLds::KT;
    unsigned char* const ktlb = lds + ScanLds::KTL;
    const float* gr = reinterpret_cast<const float*>(lds + ScanLds::GR);

    // The wave index is read from lane 0 so that the compiler treats it, and
    // what derives from it (the side, the step tile), as wave-uniform.
    const uint32_t tid = threadIdx.x, l = tid & 63u, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t lr = l & 15u, lg = l >> 4;
    const uint32_t tt = w & 3u;                         // step tile
    const bool qside = w >= 4u;
    const uint32_t slices = Dv / kRows;
    // Workgroup order: (b, key head, value head of the key head, row block),
    // renumbered so each XCD takes a contiguous range: the row blocks of a
    // head, and the value heads that read one key head's rows, share an L2.
    uint32_t li = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const uint32_t dv0 = (li % slices) * kRows;
    li /= slices;
    const uint32_t j = li % group;
    li /= group;
    const uint32_t hk = li % Hk, b = li / Hk;
    const uint32_t hv = tiled ? hk + Hk * j : hk * group + j;
    const uint32_t n = b * Hv + hv;                     // b * Hv + hv

    // This lane's 16-byte state piece: row dv0 + lr, columns kcol(w, 4 lg) .. +3
    // (the key index is permuted, see kcol); with 192 key columns waves 4-7
    // also hold tile w2 = w + 4.
    const bool extra = DK == 192 && w >= 4u;
    const uint32_t w2 = w + 4u;
    const size_t srow = (static_cast<size_t>(n) * Dv + dv0 + lr) * DK + kcol(w, 4u * lg);
    const size_t srow2 = (static_cast<size_t>(n) * Dv + dv0 + lr) * DK + kcol(w2, 4u * lg);
    f32x4v acc, acc2 = {0.f, 0.f, 0.f, 0.f};
    {
        const float4 s4 = *reinterpret_cast<const float4*>(state_in + srow);
        acc = f32x4v{s4.x, s4.y, s4.z, s4.w};
        if (extra) {
            const float4 t4 = *reinterpret_cast<const float4*>(state_in + srow2);
            acc2 = f32x4v{t4.x, t4.y, t4.z, t4.w};
        }
    }

    void* out = qside ? y : delta_log;                  // what this wave writes (delta_log may be NULL)
    const unsigned char* wsn = ws + static_cast<size_t>(n) * nchunks * PrefillWs::kBytes;
    // This lane's row of the A operand of X (K on the K side, Q on the Q side):
    // step 16 tt + lr, key columns 32 m + 8 lg .. +7 for m = 0..3, i.e. the
    // fragments of key steps 2m and 2m+1, read straight from the input.
    const char* arow = static_cast<const char*>(qside ? q : k) + (static_cast<size_t>(b) * T * Hk + hk) * (DK * 2) +
                       lg * 16;
    const size_t arow_step = static_cast<size_t>(Hk) * DK * 2;      // bytes per step
    const char* a_lane = arow + (16u * tt + lr) * arow_step;
    const char* a_last = arow + static_cast<size_t>(T - 1) * arow_step;
    auto aload = [&](u32x4 (&a)[NB], uint32_t t0n) {
        const char* src = t0n + 16u * tt + lr < T ? a_lane + t0n * arow_step : a_last;
#pragma unroll
        for (int m = 0; m < NB; ++m) a[m] = *reinterpret_cast<const u32x4*>(src + m * 64);
    };
    // Tb (K side) or P (Q side) fragments of step tile tt: up to four 16-byte
    // slots per lane (hi, lo), loaded from the workspace two chunks ahead.
    // m[2 kb] = hi, m[2 kb + 1] = lo part of step block kb; block 1 only for
    // step tiles 2 and 3 (it is zero for tiles 0 and 1).
    const bool upper = tt >= 2u;
    const size_t mfrag = (qside ? PrefillWs::kP : PrefillWs::kTb) + static_cast<size_t>(tt) * 2 * 2048 + l * 16;
    auto mload = [&](u32x4 (&m)[4], uint32_t cc) {
        const unsigned char* base = wsn + cc * static_cast<size_t>(PrefillWs::kBytes) + mfrag;
        m[0] = *reinterpret_cast<const u32x4*>(base);
        m[1] = *reinterpret_cast<const u32x4*>(base + kFragLo);
        if (upper) {
            m[2] = *reinterpret_cast<const u32x4*>(base + 2048);
            m[3] = *reinterpret_cast<const u32x4*>(base + 2048 + kFragLo);
        }
    };

    // Staging loads.  Every thread issues the same two loads (threads with
    // nothing to fetch read a valid address and drop the value), so that the
    // number of memory operations in flight does not depend on the lane and
    // the waits for them can be placed exactly where the data is used.
    // Per-lane base pointers are formed once; a chunk adds a wave-uniform
    // offset, and a row past T reads row T-1 instead.  Without a mask the
    // mask word is read from k (B*T*Hk*Dk/2 words cover every index).
    const size_t rs = static_cast<size_t>(Hv) * Dv;                 // elements per step of v, y, delta
    const bool vthread = tid >= 32u && tid < 160u;
    const uint32_t vhalf = (tid - 32u) & 1u;
    const uint32_t mrow = vthread ? (tid - 32u) >> 1 : (tid >= 160u && tid < 224u ? tid - 160u : 0u);
    const size_t vhead = (static_cast<size_t>(b) * T * Hv + hv) * Dv + dv0 + vhalf * 8;
    const uint16_t* v_lane = static_cast<const uint16_t*>(v) + vhead + mrow * rs;
    const uint16_t* v_last = static_cast<const uint16_t*>(v) + vhead + static_cast<size_t>(T - 1) * rs;
    const uint32_t* mwords = (mask ? mask : static_cast<const uint32_t*>(k)) + static_cast<size_t>(b) * T;
    const unsigned char* g_lane = wsn + PrefillWs::kGamma + (tid & 31u) * 16;
    auto sload = [&](ScanStage& st, uint32_t cc) {
        const uint32_t t0n = cc * kC;
        const bool in = t0n + mrow < T;
        const unsigned char* vsrc = reinterpret_cast<const unsigned char*>(in ? v_lane + t0n * rs : v_last);
        const unsigned char* src = vthread ? vsrc : g_lane + cc * static_cast<size_t>(PrefillWs::kBytes);
        st.gv = *reinterpret_cast<const u32x4*>(src);
        // The raw word: selecting on it here would wait for the load (the
        // select is made where the word is used, in stage_store).
        st.mv = mwords[in ? t0n + mrow : T - 1];
    };
    ScanStage sta, stb;
    u32x4 mfa[4] = {}, mfb[4] = {}, aka[NB], akb[NB];
    {
        const uint32_t c1 = nchunks > 1u ? 1u : 0u;
        sload(sta, 0u);
        sload(stb, c1);
        mload(mfa, 0u);
        mload(mfb, c1);
    }
    aload(aka, 0u);
    aload(akb, (nchunks > 1u ? 1u : 0u) * kC);
    // One pending output tile per wave (Delta of this chunk on the K side, Y of
    // the previous chunk on the Q side), stored in the next iteration just
    // before its loads are issued.  The tile goes through this wave's own LDS
    // area as bf16 with a flag per row, so that each lane stores one 8-byte
    // piece (four consecutive values of one step) instead of four 2-byte
    // values of four steps.  Only this wave touches its area, in program order.
    uint16_t* const ot = reinterpret_cast<uint16_t*>(lds + ScanLds::OT) + w * 256;
    uint32_t* const otf = reinterpret_cast<uint32_t*>(lds + ScanLds::OTF) + w * 16;
    bool pend_valid = false;
    uint32_t pend_t0 = 0u;
    // The state update's A operand of key tile ks over steps 32 kb .. 32 kb + 31:
    // lane (lr, lg) gets K[32 kb + 8 lg + j][kcol(ks, lr)], j = 0..7, from two
    // transposing reads of the row-major keys.  Lane lr addresses row
    // 32 kb + 8 lg + lr / 4 (then the row 4 below) at the four columns
    // kcol(ks, 4 (lr % 4) .. + 3), which are consecutive; the read hands lane
    // lr column kcol(ks, lr) of the four rows its group addressed.
    auto kt_frag = [&](const unsigned char* base, uint32_t ks, uint32_t kb) {
        const uint32_t t = 32u * kb + 8u * lg + (lr >> 2);   // t / 8 and (t + 4) / 8 have the parity of lg
        const uint32_t piece = 4u * (ks >> 1) + (lr & 3u);    // 16-byte piece of columns 8 piece ..
        const unsigned char* p = base + t * ScanLds::KRS + piece * 16u + (((ks ^ lg) & 1u) * 8u);
        const u32x2 a = lds_read_tr16(p), b = lds_read_tr16(p + 4u * ScanLds::KRS);
        return u32x4{a.x, a.y, b.x, b.y};
    };
    auto produce = [&](const f32x4v& vals, uint32_t actbits, uint32_t t0p) {
        if constexpr (IO == kBF16) {
            // Round to nearest even with the packed conversion; a NaN is
            // replaced by the canonical quiet NaN first, so the bits equal
            // f32_to_bf16_bits' (NaN -> 0x7FC0).
            f32x4v v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = vals[r] != vals[r] ? __uint_as_float(0x7fc00000u) : vals[r];
            const uint32_t p01 = cvt_pk_bf16(v[0], v[1]), p23 = cvt_pk_bf16(v[2], v[3]);
            ot[(4u * lg + 0) * 16 + lr] = static_cast<uint16_t>(p01);
            ot[(4u * lg + 1) * 16 + lr] = static_cast<uint16_t>(p01 >> 16);
            ot[(4u * lg + 2) * 16 + lr] = static_cast<uint16_t>(p23);
            ot[(4u * lg + 3) * 16 + lr] = static_cast<uint16_t>(p23 >> 16);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) ot[(4u * lg + r) * 16 + lr] = static_cast<uint16_t>(f32_to_f16_bits(vals[r]));
        }
        if (lr == 0u) {
#pragma unroll
            for (int r = 0; r < 4; ++r) otf[4u * lg + r] = (actbits >> r) & 1u;
        }
        pend_valid = true;
        pend_t0 = t0p;
    };
    // This lane's 8-byte piece: step 16 tt + l / 4 of a chunk starting at step
    // 0, values dv0 + 4 (l % 4) .. +3; a chunk adds a wave-uniform offset.
    uint16_t* const out_lane = out == nullptr ? nullptr
        : static_cast<uint16_t*>(out) + (static_cast<size_t>(b) * T * Hv + hv) * Dv + dv0 + 4u * (l & 3u) +
              (16u * tt + (l >> 2)) * rs;
    auto flush = [&]() {
        if (out == nullptr || !pend_valid) return;
        const u32x2 piece = *reinterpret_cast<const u32x2*>(ot + (l >> 2) * 16 + 4u * (l & 3u));
        if (otf[l >> 2] != 0u) *reinterpret_cast<u32x2*>(out_lane + pend_t0 * rs) = piece;
        pend_valid = false;
    };
    // Q side: what Y of a chunk needs one iteration later.
    f32x4v xq_prev = {0.f, 0.f, 0.f, 0.f}, gam_prev = xq_prev;
    u32x4 p_prev[4];
    uint32_t act_prev = 0u;
    auto y_tile = [&](const unsigned char* dsrc) -> f32x4v {
        f32x4v Y, Y2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) Y[r] = gam_prev[r] * xq_prev[r];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb == 1 && !upper) break;
            const u32x4 dh = bop_hi(dsrc, kb, l), dl = bop_lo(dsrc, kb, l);
            Y = mfma_bf16_k32(p_prev[2 * kb], dh, Y);
            Y2 = mfma_bf16_k32(p_prev[2 * kb], dl, Y2);
            Y2 = mfma_bf16_k32(p_prev[2 * kb + 1], dh, Y2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Y[r] += Y2[r];
        return Y;
    };

    // One chunk.  st, mf and ak hold its staged rows, its Tb or P fragments
    // and its key or query fragments; each then receives those of the chunk
    // after next, once this chunk is done with it.  The loop below runs two
    // chunks per iteration with the buffers swapped, so that no register still
    // being loaded is copied (a copy would wait for the load) and every load
    // has one to two chunks of compute to arrive in.
    auto chunk = [&](uint32_t c, ScanStage& st, u32x4 (&mf)[4], u32x4 (&ak)[NB])
                     __attribute__((always_inline)) {
        const uint32_t t0 = c * kC;
        // (Past the last chunk the loads repeat it and go unused, so that
        // every iteration issues the same memory operations.)
        const uint32_t c2 = c + 2 < nchunks ? c + 2 : nchunks - 1;
        stage_store<ScanLds>(st, mask != nullptr, lds, T, t0, tid);
        {
            u32x2 hi, lo;
            split4(acc, hi, lo);
            // hi parts of key tiles 2m and 2m+1 side by side in slot m, lo
            // parts in slot NB + m: one 16-byte read is then a B operand of
            // the 32-deep product over key columns 32m .. 32m + 31.
            *reinterpret_cast<u32x2*>(reinterpret_cast<unsigned char*>(&sfr[w >> 1][l]) + (w & 1u) * 8) = hi;
            *reinterpret_cast<u32x2*>(reinterpret_cast<unsigned char*>(&sfr[NB + (w >> 1)][l]) + (w & 1u) * 8) = lo;
            if (extra) {
                split4(acc2, hi, lo);
                *reinterpret_cast<u32x2*>(reinterpret_cast<unsigned char*>(&sfr[w2 >> 1][l]) + (w2 & 1u) * 8) = hi;
                *reinterpret_cast<u32x2*>(reinterpret_cast<unsigned char*>(&sfr[NB + (w2 >> 1)][l]) + (w2 & 1u) * 8) =
                    lo;
            }
        }
        __syncthreads();

        uint32_t act;                                   // bit r: step 16 tt + 4 lg + r is active
        {
            const u32x4 f = *reinterpret_cast<const u32x4*>(lds + ScanLds::AF + (16u * tt + 4u * lg) * 4);
            act = f.x | (f.y << 1) | (f.z << 2) | (f.w << 3);
        }

        // X = (K or Q) S0^T for step tile tt (hi and lo parts apart).  The row
        // of an inactive step is zero (a select, so a NaN there cannot enter).
        // Lane (lr, lg) holds key columns 32m + 8lg .. +7 of its row for each
        // m: the A operand of the 32-deep product over columns 32m .. 32m + 31.
        // fp16 rows: a8 holds the hi and a8l the lo bf16 parts.
        u32x4 a8[NB], a8l[NB];
        {
            const bool ra = reinterpret_cast<const uint32_t*>(lds + ScanLds::AF)[16u * tt + lr] != 0u;
            const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                a8[m] = ra ? ak[m] : z;
                if constexpr (IO == kF16) split_f16x8(a8[m], a8[m], a8l[m]);
            }
        }
        // The previous chunk's outputs and the loads for the chunk after next
        // are issued here, behind the first barrier and before the products
        // below, so that the vector-memory path works while the matrix cores
        // do (issued after the products, they held up R by ~8 µs per launch).
        flush();
        sload(st, c2);                                  // st was stored into LDS at the top
        aload(ak, c2 * kC);                             // ak is free again: its selects are done
        f32x4v x = {0.f, 0.f, 0.f, 0.f}, x2 = x;
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const u32x4 sh = sfr[m][l], sl = sfr[NB + m][l];
            x = mfma_bf16_k32(a8[m], sh, x);
            x2 = mfma_bf16_k32(a8[m], sl, x2);
            if constexpr (IO == kF16) x2 = mfma_bf16_k32(a8l[m], sh, x2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] += x2[r];
        f32x4v gam;
        {
            const float4 g4 = *reinterpret_cast<const float4*>(gr + 16u * tt + 4u * lg);
            gam = f32x4v{g4.x, g4.y, g4.z, g4.w};
        }
        if (!qside) {
            // This wave's 16 key rows into LDS as they are (natural key
            // order), one 16-byte piece per block; the state update reads them
            // transposed (kt_frag).
            const bool swap = (lr & 8u) != 0u;                // row 16 tt + lr in an odd 8-row group
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                const uint32_t o = (16u * tt + lr) * ScanLds::KRS + (32u * m + 8u * lg) * 2u;
                const u32x4 v = a8[m];
                *reinterpret_cast<u32x4*>(ktb + o) = swap ? u32x4{v.z, v.w, v.x, v.y} : v;
                if constexpr (IO == kF16) {
                    const u32x4 vl = a8l[m];
                    *reinterpret_cast<u32x4*>(ktlb + o) = swap ? u32x4{vl.z, vl.w, vl.x, vl.y} : vl;
                }
            }
            const uint16_t* vr = reinterpret_cast<const uint16_t*>(lds + ScanLds::VR);
            f32x4v R;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                R[r] = in_f32<IO>(vr[(16u * tt + 4u * lg + r) * 16 + lr]) - gam[r] * x[r];
            u32x2 hi, lo;
            split4(R, hi, lo);
            bop_store(rfr, tt, lr, lg, hi, lo);
        }
        __syncthreads();

        if (!qside) {
            // Delta (step tile tt) = Tb R.  Tb is zero above the diagonal, so
            // the tiles past tt add exact zeros (block 1 is skipped for tiles
            // 0 and 1).
            f32x4v D = {0.f, 0.f, 0.f, 0.f}, D2 = D;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb == 1 && !upper) break;
                const u32x4 rh = bop_hi(rfr, kb, l), rl = bop_lo(rfr, kb, l);
                D = mfma_bf16_k32(mf[2 * kb], rh, D);
                D2 = mfma_bf16_k32(mf[2 * kb], rl, D2);
                D2 = mfma_bf16_k32(mf[2 * kb + 1], rh, D2);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) D[r] += D2[r];
            u32x2 hi, lo;
            split4(D, hi, lo);
            bop_store(dfr + (c & 1u) * ScanLds::BOP, tt, lr, lg, hi, lo);
            f32x4v Dt;
            const float4 r4 = *reinterpret_cast<const float4*>(gr + kC + 16u * tt + 4u * lg);
            Dt[0] = r4.x * D[0]; Dt[1] = r4.y * D[1]; Dt[2] = r4.z * D[2]; Dt[3] = r4.w * D[3];
            split4(Dt, hi, lo);
            bop_store(dtf, tt, lr, lg, hi, lo);
            produce(D, act, t0);
        } else {
            if (c > 0) {
                // Y of the previous chunk = gamma o X_Q + P Delta.
                produce(y_tile(dfr + ((c - 1) & 1u) * ScanLds::BOP), act_prev, t0 - kC);
            }
            xq_prev = x;
            gam_prev = gam;
            act_prev = act;
#pragma unroll
            for (int i = 0; i < 4; ++i) p_prev[i] = mf[i];      // P of this chunk, for its Y next iteration
        }
        const float gC = gr[kC - 1];
        __syncthreads();

        // S^T <- gamma_63 S^T + K^T (rho o Delta) for this wave's key tiles.
        f32x4v lo_acc = {0.f, 0.f, 0.f, 0.f}, lo_acc2 = lo_acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc[r] *= gC;
            acc2[r] *= gC;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const u32x4 dh = bop_hi(dtf, kb, l), dl = bop_lo(dtf, kb, l);
            const u32x4 a = kt_frag(ktb, w, kb);
            acc = mfma_bf16_k32(a, dh, acc);
            lo_acc = mfma_bf16_k32(a, dl, lo_acc);
            if constexpr (IO == kF16) lo_acc = mfma_bf16_k32(kt_frag(ktlb, w, kb), dh, lo_acc);
            if (extra) {
                const u32x4 a2 = kt_frag(ktb, w2, kb);
                acc2 = mfma_bf16_k32(a2, dh, acc2);
                lo_acc2 = mfma_bf16_k32(a2, dl, lo_acc2);
                if constexpr (IO == kF16) lo_acc2 = mfma_bf16_k32(kt_frag(ktlb, w2, kb), dh, lo_acc2);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc[r] += lo_acc[r];
            acc2[r] += lo_acc2[r];
        }
        mload(mf, c2);                                  // mf's last use was before the third barrier
    };
    uint32_t c = 0;
    for (; c + 1 < nchunks; c += 2) {
        chunk(c, sta, mfa, aka);
        chunk(c + 1, stb, mfb, akb);
    }
    if (c < nchunks) chunk(c, sta, mfa, aka);          // an odd chunk count's last chunk

    flush();
    if (qside) {
        // Y of the last chunk (its Delta fragments were written before the
        // last iteration's final barrier).
        produce(y_tile(dfr + ((nchunks - 1) & 1u) * ScanLds::BOP), act_prev, (nchunks - 1) * kC);
        flush();
    }
    *reinterpret_cast<float4*>(state_out + srow) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    if (extra) *reinterpret_cast<float4*>(state_out + srow2) = make_float4(acc2[0], acc2[1], acc2[2], acc2[3]);
}

}  // namespace

uint64_t prefill_workspace_bytes(uint32_t B, uint32_t T, uint32_t Hv) {
    const uint64_t nchunks = (static_cast<uint64_t>(T) + kC - 1) / kC;
    uint64_t n = static_cast<uint64_t>(B) * Hv, bytes;    // B * Hv fits in 64 bits
    if (__builtin_mul_overflow(n, nchunks, &n) || __builtin_mul_overflow(n, uint64_t(PrefillWs::kBytes), &bytes))
        return ~uint64_t(0);
    return bytes;
}

// ------------------------------------------------ allocation-free variant

// The workspace of gdn_prefill_noalloc.  Each GPU the library runs on holds
// its own copy from the first call until the process ends, and every call of
// that entry point on a GPU shares it.  prep writes every byte of a block
// that scan reads, so nothing here has to start at zero.  In host code the
// name `scratch` is only a stand-in for the symbol, not a device address:
// kernels get the address prefill_scratch() looked up.
static_assert(kPrefillScratchBytes == 2048ull * PrefillWs::kBytes, "scratch size");
static __device__ __align__(256) unsigned char scratch[kPrefillScratchBytes];

hipError_t prefill_scratch(hipStream_t stream, void** out) {
    constexpr int kDevices = 64;
    static std::atomic<void*> addr[kDevices];
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    hipDevice_t sdev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return e;
    }
    if (sdev != cur || cur < 0 || cur >= kDevices) return hipErrorInvalidDevice;
    void* p = addr[cur].load(std::memory_order_acquire);
    if (p == nullptr) {
        // once per device, with that device current (two threads racing here
        // both store the same address)
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[cur].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

bool prefill_supported(uint32_t Dk, uint32_t Dv, int io) {
    return (io == kBF16 || io == kF16) && (Dk == 128 || Dk == 192) && Dv % kRows == 0;
}

namespace {

template <int IO, int DK>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    using PL = PrepLds<DK>;
    using SL = ScanLds<IO, DK>;
    const uint32_t nchunks = (a.T + kC - 1) / kC;
    const uint32_t group = a.Hv / a.Hk;
    const int tiled = a.map == 1;
    auto* ws = static_cast<unsigned char*>(a.workspace);
    // Both kernels take more than the default 64 KiB of LDS: raise their
    // limits once per device.
    static std::atomic<uint64_t> lds_set{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
    if (bit == 0 || !(lds_set.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_prefill_scan_kernel<IO, DK>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, SL::BYTES);
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_prefill_prep_kernel<IO, DK>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, PL::BYTES);
        if (e != hipSuccess) return e;
        lds_set.fetch_or(bit, std::memory_order_release);
    }
    const uint32_t head_sets = (group + kPrepHeads - 1) / kPrepHeads;
    hipLaunchKernelGGL((gdn_prefill_prep_kernel<IO, DK>), dim3(a.B * a.Hk * nchunks * head_sets), dim3(256), PL::BYTES,
                       stream, a.q, a.k, a.g, a.beta, a.mask, ws, a.k_log, a.g_log, a.T, a.Hk, a.Hv, nchunks, group,
                       head_sets, tiled);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_prefill_scan_kernel<IO, DK>), dim3(a.B * a.Hv * (a.Dv / kRows)), dim3(512), SL::BYTES,
                       stream, a.q, a.k, a.v, a.state_in, a.mask, ws, a.y, a.state_out, a.delta_log, a.T, a.Hk,
                       a.Hv, a.Dv, nchunks, group, tiled);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.io == kBF16) return a.Dk == 128 ? launch_prefill_t<kBF16, 128>(a, stream) : launch_prefill_t<kBF16, 192>(a, stream);
    return a.Dk == 128 ? launch_prefill_t<kF16, 128>(a, stream) : launch_prefill_t<kF16, 192>(a, stream);
}

}  // namespace gdn
