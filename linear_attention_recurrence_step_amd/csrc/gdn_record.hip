// gdn_record: gated delta-rule forward step with innovation-tape capture, gfx950.
//
// What it computes is the record kernel (macro `gated_delta_record!`) of the
// metaltile-std 0.1.0 page src/ffai/gated_delta_replay.rs: per (b, hv, dv) row
// and active step t, decay the row by g, read it out against k, form the
// innovation delta = (v - kv) * beta, write delta to the tape, add delta * k to
// the row and read the updated row out against q into y.
//
// The read-outs are evaluated as
//     kv = g (S . k),   y = g (S . q) + delta * (k . q),
// which equal (g S) . k and (g S + delta k^T) . q exactly in real arithmetic
// and let both dot products run in one pass over the row before its decay;
// only the rounding differs (within the stated tolerances).
//
// How it maps onto CDNA4 (not the page's one-32-lane-group-per-row layout):
//  * 16 lanes (one DPP row) share a state row; lane l holds the Dk/16 columns
//    {(c*16 + l)*W + w}, so every 16-lane vector access is contiguous.
//  * A thread owns RPT consecutive rows of one head; a workgroup of NT threads
//    covers R = RPT*NT/16 consecutive rows.  The rows stay in VGPRs for all T
//    steps; the state is read once and written once (non-temporal) per launch.
//  * Dot products finish with a 4-stage DPP butterfly inside the 16-lane row
//    (no LDS, no barrier); independent sums are reduced stage-interleaved.
//  * One step (T = 1, decode): the direct kernel loads k, q, v, g, beta per
//    lane straight from global memory (the repeats of a key vector across rows
//    hit the L1/L2).
//  * Several steps: the staged kernel brings the inputs of a chunk of steps
//    into LDS in one round of coalesced loads, prefetches the next chunk into
//    registers while computing, and buffers y and delta of the chunk in LDS so
//    they leave as vector stores.
//  * The mask row [B, T] is uniform over a workgroup, so inactive steps are a
//    scalar branch around the whole step and write nothing.
//  * Optional tape capture: the first row group of each head also copies the
//    raw bits of the step's keys (expanded to the value head) and gate into
//    k_log and g_log, so the replay's tape needs no separate pass.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

#include <atomic>

namespace gdn {
namespace {

// This lane's part of a Dk-length dot product over its E columns, in a fixed
// order shared by every kernel that needs it: two interleaved partial sums
// (even and odd columns) added at the end, so the dependent chain is E/2
// fused multiply-adds long.
template <int E>
__device__ __forceinline__ float lane_dot(const float (&x)[E], const float (&y)[E]) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int e = 0; e + 1 < E; e += 2) {
        a = fmaf(x[e], y[e], a);
        b = fmaf(x[e + 1], y[e + 1], b);
    }
    if constexpr (E % 2 == 1) a = fmaf(x[E - 1], y[E - 1], a);
    return a + b;
}

// One active step on the RPT rows this lane holds (E columns of each):
// read-outs against k and q, innovation, decay and rank-1 write.  The
// read-outs are taken on the row before the decay and scaled by the gate
// afterwards, kv = g (S . k) and (g S) . q = g (S . q), which equal the
// read-outs of the decayed row in real arithmetic and take the decay off the
// step-to-step dependence chain; the state update itself is
// S <- fma(k, delta, S * g), the same two roundings as the replay's fold.
// kq = k . q of the step.  d and out receive the innovation and the output of
// every row (identical bits in all 16 lanes of the row).
template <int RPT, int E>
__device__ __forceinline__ void record_step(float (&s)[RPT][E], const float (&kk)[E],
                                            const float (&qq)[E], const float (&vv)[RPT],
                                            float gt, float beta, float kq, float (&d)[RPT],
                                            float (&out)[RPT]) {
    float red[2 * RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        red[r] = lane_dot<E>(s[r], kk);                              // S . k
        red[RPT + r] = lane_dot<E>(s[r], qq);                        // S . q
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) s[r][e] = s[r][e] * gt;          // decay, off the chain
    row16_sum_n<2 * RPT>(red);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        d[r] = (vv[r] - gt * red[r]) * beta;
        out[r] = fmaf(d[r], kq, gt * red[RPT + r]);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) s[r][e] = fmaf(kk[e], d[r], s[r][e]);   // rank-1 write
}

// ------------------------------------------------------------ direct kernel

// One step (T = 1, decode).  Every input of the step (k, q, v, g, beta and
// the mask word) is issued right behind the state loads, so the kernel
// waits for memory once; there is no step loop, whose loop-carried state
// registers had made the compiler wait for the state before issuing the
// step's loads.  An inactive step leaves the state as loaded and writes
// nothing.
template <int IO, int DK, int RPT, int NT>
__global__ __launch_bounds__(NT) void gdn_record_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ g, const void* __restrict__ beta,
    const float* state_in, const uint32_t* __restrict__ mask,
    void* __restrict__ y, float* state_out, void* __restrict__ delta_log,
    void* __restrict__ k_log, void* __restrict__ g_log,
    uint32_t Hk, uint32_t Hv, uint32_t Dv, uint32_t row_blocks, int tiled)
{
    constexpr int L = 16;                 // lanes per state row
    constexpr int E = DK / L;             // state values per lane per row
    constexpr int W = E < 4 ? E : 4;      // columns per contiguous chunk
    constexpr int NC = E / W;             // chunks per lane
    constexpr int SLOTS = NT / L;         // row groups per workgroup
    constexpr int R = SLOTS * RPT;        // rows per workgroup
    static_assert(DK % (L * W) == 0 && NC * W == E, "unsupported Dk");

    const uint32_t lane = threadIdx.x & (L - 1);
    const uint32_t slot = threadIdx.x / L;

    // Workgroup blk covers rows [blk*R, blk*R + R) of the flattened
    // [B*Hv*Dv] row space (R divides Dv, so they belong to one head).  The
    // state address needs no division, so the state loads go out first and
    // the head arithmetic below overlaps their latency.
    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const size_t srow = (static_cast<size_t>(blk) * R + slot * RPT) * DK;

    float s[RPT][E];
    load_state_rows<RPT, E>(state_in + srow, lane, s);

    const uint32_t n = blk / row_blocks;                      // b * Hv + hv (= bt * Hv + hv: T = 1)
    const uint32_t row0 = (blk - n * row_blocks) * R + slot * RPT;  // first row within the head
    const uint32_t b = n / Hv;
    const uint32_t hv = n - b * Hv;
    const uint32_t hk = tiled ? hv % Hk : hv / (Hv / Hk);
    const size_t kq = (static_cast<size_t>(b) * Hk + hk) * DK;
    const size_t vo = static_cast<size_t>(n) * Dv + row0;

    RawIo<IO, W> kr[NC], qr[NC];
    RawIo<IO, RPT> vr;
    RawIo<IO, 1> gr, br;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        kr[c].load(k, kq + (c * L + lane) * W);
        qr[c].load(q, kq + (c * L + lane) * W);
    }
    vr.load(v, vo);
    gr.load(g, n);
    br.load(beta, n);
    const bool active = mask == nullptr || mask[b] != 0u;

    // One exit: an inactive step (no decay, no writes) falls through to the
    // state store.  (An early return there was structurized into a cycle
    // whose loop-invariant code motion dropped the non-temporal hint from
    // the state stores.)
    if (active) {
        if (row0 == 0) {                                      // tape capture: bit copies
            if (k_log != nullptr)
#pragma unroll
                for (int c = 0; c < NC; ++c) kr[c].store(k_log, static_cast<size_t>(n) * DK + (c * L + lane) * W);
            if (g_log != nullptr && lane == 0) gr.store(g_log, n);
        }
        float kk[E], qq[E], vv[RPT];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int w = 0; w < W; ++w) {
                kk[c * W + w] = kr[c].at(w);
                qq[c * W + w] = qr[c].at(w);
            }
#pragma unroll
        for (int r = 0; r < RPT; ++r) vv[r] = vr.at(r);
        float kqs[1] = {lane_dot<E>(kk, qq)};
        row16_sum_n<1>(kqs);
        float d[RPT], out[RPT];
        record_step<RPT, E>(s, kk, qq, vv, gr.at(0), br.at(0), kqs[0], d, out);
        if (delta_log != nullptr && lane == 0) io_store_vec<IO, RPT>(delta_log, vo, d);
        if (lane == 0) io_store_vec<IO, RPT>(y, vo, out);
    }

    store_state_rows<RPT, E>(state_out + srow, lane, s);
}

// ------------------------------------------------------ short-tape kernel

// Tapes of at most this many steps run the short-tape kernel.
constexpr uint32_t kShortDirectSteps = 4;

// Record of a short tape (2 <= T <= TMAX), the speculative-decode case: the
// direct kernel's layout, with every step's inputs loaded right after the
// state (step indices past T clamped to T - 1, so every load is valid and
// unconditional) and the steps then run from registers: no LDS, no barrier,
// and a single round trip to memory before the first step.  k . q of every
// step is reduced once up front, off the state's chain.  Same arithmetic as
// the other record kernels (record_step), so the same bits.
template <int IO, int DK, int RPT, int NT, int TMAX>
__global__ __launch_bounds__(NT) void gdn_record_short_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ g, const void* __restrict__ beta,
    const float* state_in, const uint32_t* __restrict__ mask,
    void* __restrict__ y, float* state_out, void* __restrict__ delta_log,
    void* __restrict__ k_log, void* __restrict__ g_log,
    uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dv, uint32_t row_blocks, int tiled)
{
    constexpr int L = 16;
    constexpr int E = DK / L;
    constexpr int W = E < 4 ? E : 4;
    constexpr int NC = E / W;
    constexpr int SLOTS = NT / L;
    constexpr int R = SLOTS * RPT;
    static_assert(DK % (L * W) == 0 && NC * W == E, "unsupported Dk");

    const uint32_t lane = threadIdx.x & (L - 1);
    const uint32_t slot = threadIdx.x / L;
    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const size_t srow = (static_cast<size_t>(blk) * R + slot * RPT) * DK;

    float s[RPT][E];
    load_state_rows<RPT, E>(state_in + srow, lane, s);

    const uint32_t n = blk / row_blocks;                      // b * Hv + hv
    const uint32_t row0 = (blk - n * row_blocks) * R + slot * RPT;
    const uint32_t b = n / Hv;
    const uint32_t hv = n - b * Hv;
    const uint32_t hk = tiled ? hv % Hk : hv / (Hv / Hk);

    RawIo<IO, W> kr[TMAX][NC], qr[TMAX][NC];
    RawIo<IO, RPT> vr[TMAX];
    RawIo<IO, 1> gr[TMAX], br[TMAX];
    uint32_t mk[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        const uint32_t tc = static_cast<uint32_t>(t) < T ? static_cast<uint32_t>(t) : T - 1;
        const size_t bt = static_cast<size_t>(b) * T + tc;
        const size_t kq = (bt * Hk + hk) * DK;
        const size_t gi = bt * Hv + hv;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            kr[t][c].load(k, kq + (c * L + lane) * W);
            qr[t][c].load(q, kq + (c * L + lane) * W);
        }
        vr[t].load(v, gi * Dv + row0);
        gr[t].load(g, gi);
        br[t].load(beta, gi);
        mk[t] = mask != nullptr ? mask[bt] : 1u;
    }

    auto widen = [&](const RawIo<IO, W> (&raw)[NC], float (&out)[E]) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int w = 0; w < W; ++w) out[c * W + w] = raw[c].at(w);
    };
    float kq[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        float kk[E], qq[E];
        widen(kr[t], kk);
        widen(qr[t], qq);
        kq[t] = lane_dot<E>(kk, qq);
    }
    row16_sum_n<TMAX>(kq);

    const bool capture = row0 == 0;                           // first row group of the head
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (static_cast<uint32_t>(t) >= T) break;
        if (mk[t] == 0u) continue;                            // inactive step: no decay, no writes
        const size_t bt = static_cast<size_t>(b) * T + t;
        const size_t gi = bt * Hv + hv;
        const size_t vo = gi * Dv + row0;
        if (capture) {                                        // tape capture: bit copies
            if (k_log != nullptr)
#pragma unroll
                for (int c = 0; c < NC; ++c) kr[t][c].store(k_log, gi * DK + (c * L + lane) * W);
            if (g_log != nullptr && lane == 0) gr[t].store(g_log, gi);
        }
        float kk[E], qq[E], vv[RPT];
        widen(kr[t], kk);
        widen(qr[t], qq);
#pragma unroll
        for (int r = 0; r < RPT; ++r) vv[r] = vr[t].at(r);
        float d[RPT], out[RPT];
        record_step<RPT, E>(s, kk, qq, vv, gr[t].at(0), br[t].at(0), kq[t], d, out);
        if (delta_log != nullptr && lane == 0) io_store_vec<IO, RPT>(delta_log, vo, d);
        if (lane == 0) io_store_vec<IO, RPT>(y, vo, out);
    }

    store_state_rows<RPT, E>(state_out + srow, lane, s);
}

// ------------------------------------------------------------ staged kernel

// Chunk lengths of the staged kernel: the inputs of up to TC steps sit in LDS
// at once (as float32), and the next chunk's loads wait in registers.  A
// longer chunk pays its barriers and staging over more steps but costs LDS
// and registers, so the length follows the launch: 8 (short tapes), 16 (up to
// 16 steps), 32 (16 at Dk above 128) for long tapes, and 64 for long tapes
// whose grid leaves each CU at most one workgroup (a prefill over few heads),
// where occupancy is not at stake.
template <int DK>
constexpr int staged_chunk() { return DK <= 128 ? 32 : 16; }
constexpr int kMediumChunk = 16;
constexpr int kWideChunk = 64;

// Steps whose LDS operands are read together; LDS chunks are padded to a
// multiple of this many rows.
constexpr int kGroup = 4;

// Tapes of at most this many steps run the short configuration of the staged
// kernel (one chunk of this length, operands read one step at a time).
constexpr uint32_t kShortChunk = 8;

// LDS rows of a chunk: min(TC, T) rounded up to a whole group.
__host__ __device__ constexpr uint32_t chunk_alloc_rows(uint32_t tc, uint32_t T) {
    const uint32_t r = T < tc ? T : tc;
    return (r + kGroup - 1) / kGroup * kGroup;
}

// LDS floats for a chunk of `rows` steps: k and q rows, the step scalars
// (g, beta, k.q, mask), this group's v, and two buffers of interleaved
// (y, delta) pairs plus an active flag per step (the previous chunk's outputs
// leave while the next chunk is computed).
__host__ __device__ constexpr size_t record_lds_floats(int rows, int dk, int r) {
    return static_cast<size_t>(rows) * (2 * dk + 4 + r + 2 * (2 * r + 1));
}

// The LDS operands of one step for one lane.
template <int E, int RPT>
struct StepOperands {
    float k[E], q[E], v[RPT];
    f32x4 sc;                                  // g, beta, k.q, mask entry (as bits)

    template <int DK, int R>
    __device__ __forceinline__ void read(const float* sk, const float* sq, const float* sv,
                                         const float* sc4, int tt, uint32_t lane, uint32_t slot) {
        constexpr int W = E < 4 ? E : 4;
#pragma unroll
        for (int c = 0; c < E / W; ++c) {
            float tk[W], tq[W];
            lds_load_vec<W>(sk + tt * DK + (c * 16 + lane) * W, tk);
            lds_load_vec<W>(sq + tt * DK + (c * 16 + lane) * W, tq);
#pragma unroll
            for (int w = 0; w < W; ++w) { k[c * W + w] = tk[w]; q[c * W + w] = tq[w]; }
        }
        lds_load_vec<RPT>(sv + tt * R + slot * RPT, v);
        sc = *reinterpret_cast<const f32x4*>(sc4 + 4 * tt);
    }
};

// Staged variant for T > 1: every step of the direct kernel would wait for its
// own inputs to arrive from memory.  Here the steps are taken in chunks of TC:
// the workgroup copies a chunk's k and q (of its key head), v (of its rows), g,
// beta and mask entries into LDS as float32 in one round of coalesced loads,
// computes k . q of each step once, and loads the following chunk into
// registers while it computes the current one from LDS.  y and delta of the
// chunk are gathered in LDS and written with vector stores after it.
// TC = kShortChunk (tapes of at most that many steps): one small chunk whose
// operands are read one step at a time, which keeps the register count (and
// so the occupancy) of this latency-bound case low.
template <int IO, int DK, int RPT, int NT, bool MASKED, int TC>
__global__ __launch_bounds__(NT) void gdn_record_staged_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ g, const void* __restrict__ beta,
    const float* state_in, const uint32_t* __restrict__ mask,
    void* __restrict__ y, float* state_out, void* __restrict__ delta_log,
    void* __restrict__ k_log, void* __restrict__ g_log,
    uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dv, uint32_t row_blocks, int tiled,
    uint32_t chunk_rows)
{
    constexpr int L = 16;
    constexpr int E = DK / L;
    constexpr int W = E < 4 ? E : 4;
    constexpr int NC = E / W;
    constexpr int SLOTS = NT / L;
    constexpr int R = SLOTS * RPT;
    constexpr bool SHORT = TC <= static_cast<int>(kShortChunk);
    constexpr int G = SHORT ? 1 : kGroup;                     // steps whose operands are read together
    constexpr int EB = IoTraits<IO>::kBytes;
    constexpr int PR = piece_elems<IO, R>();                  // v / y / delta piece (elements)
    static_assert(DK % (L * W) == 0 && NC * W == E, "unsupported Dk");
    static_assert(R <= kStagedMaxRows, "row block too large for the staged kernel");

    extern __shared__ __align__(16) float lds[];
    const int crow = static_cast<int>(chunk_rows);            // LDS rows allocated (whole groups)
    float* sk = lds;                                          // [crow][DK]
    float* sq = sk + crow * DK;                               // [crow][DK]
    float* sc = sq + crow * DK;                               // [crow][4]: g, beta, k.q, mask
    float* sv = sc + crow * 4;                                // [crow][R]
    float* obuf = sv + crow * R;                              // 2 x {(y, delta) [crow][R][2], flag [crow]}
    const int obuf_stride = crow * (2 * R + 1);

    const uint32_t lane = threadIdx.x & (L - 1);
    const uint32_t slot = threadIdx.x / L;
    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);

    // Workgroups are ordered (b, key head, value head of that key head, row
    // block), so the value heads that read one key head's q and k run next
    // to each other, on one XCD and its L2.  Under the block map that is the
    // natural head order; under the tiled map value head hv = j * Hk + hk.
    const uint32_t nord = blk / row_blocks;
    const uint32_t wrow0 = (blk - nord * row_blocks) * R;     // first row of the group in its head
    const uint32_t b = nord / Hv;
    const uint32_t hpos = nord - b * Hv;                      // position of the head in that order
    uint32_t hv = hpos, hk;
    if (tiled) {
        const uint32_t group = Hv / Hk;
        hk = hpos / group;
        hv = (hpos - hk * group) * Hk + hk;
    } else {
        hk = hpos / (Hv / Hk);
    }
    const size_t srow = ((static_cast<size_t>(b) * Hv + hv) * Dv + wrow0 + slot * RPT) * DK;

    float s[RPT][E];
    load_state_rows<RPT, E>(state_in + srow, lane, s);

    ChunkStager<IO, TC, DK, piece_elems<IO, DK>(), NT> stk, stq;
    ChunkStager<IO, TC, R, PR, NT> stv;
    ChunkStager<IO, TC, 1, 1, NT> stg, stb;
    MaskStager<TC, NT> stm;

    auto chunk_len = [&](uint32_t t0) { return static_cast<int>(T - t0 < TC ? T - t0 : TC); };
    auto load_chunk = [&](uint32_t t0) {
        const int valid = chunk_len(t0);
        const size_t bt0 = static_cast<size_t>(b) * T + t0;
        const size_t kqo = (bt0 * Hk + hk) * DK;
        stk.load(static_cast<const char*>(k) + kqo * EB, static_cast<size_t>(Hk) * DK, valid);
        stq.load(static_cast<const char*>(q) + kqo * EB, static_cast<size_t>(Hk) * DK, valid);
        stv.load(static_cast<const char*>(v) + ((bt0 * Hv + hv) * Dv + wrow0) * EB,
                 static_cast<size_t>(Hv) * Dv, valid);
        stg.load(static_cast<const char*>(g) + (bt0 * Hv + hv) * EB, Hv, valid);
        stb.load(static_cast<const char*>(beta) + (bt0 * Hv + hv) * EB, Hv, valid);
        stm.load(mask != nullptr ? mask + bt0 : nullptr, valid);
    };
    // y and delta of the chunk starting at t0 (in output buffer t0/TC mod 2),
    // from LDS to global memory in pieces of PR elements; inactive steps
    // (flag 0) are skipped.
    auto flush_chunk = [&](uint32_t t0) {
        const int valid = chunk_len(t0);
        const float* oyd = obuf + ((t0 / TC) & 1u) * obuf_stride;   // [crow][R][2]: y, delta
        const uint32_t* of = reinterpret_cast<const uint32_t*>(oyd + crow * R * 2);
        constexpr int PER_STEP = R / PR;
        for (int p = static_cast<int>(threadIdx.x); p < valid * PER_STEP; p += NT) {
            const int tt = p / PER_STEP;
            const int col = (p - tt * PER_STEP) * PR;
            if (MASKED && of[tt] == 0u) continue;
            const size_t vo = ((static_cast<size_t>(b) * T + t0 + tt) * Hv + hv) * Dv + wrow0 + col;
            float f[2 * PR], fy[PR], fd[PR];
            lds_load_vec<2 * PR>(oyd + (tt * R + col) * 2, f);
#pragma unroll
            for (int i = 0; i < PR; ++i) { fy[i] = f[2 * i]; fd[i] = f[2 * i + 1]; }
            io_store_vec<IO, PR>(y, vo, fy);
            if (delta_log != nullptr) io_store_vec<IO, PR>(delta_log, vo, fd);
        }
    };

    load_chunk(0);
    wait_vector_memory();                                     // state rows and chunk 0 are in
    for (uint32_t t0 = 0; t0 < T; t0 += TC) {
        if (t0 != 0) __syncthreads();                         // the previous chunk is computed
        const int valid = chunk_len(t0);
        float* oyd = obuf + ((t0 / TC) & 1u) * obuf_stride;   // this chunk's output buffer
        stk.store(sk, crow);
        stq.store(sq, crow);
        stv.store(sv, crow);
        // Padding rows (past the tape end, up to a whole group) become exact
        // identity steps: g = 1, beta = 0, k = q = v = 0.
        stg.store_strided(sc + 0, 4, crow, valid, 1.f);
        stb.store_strided(sc + 1, 4, crow, valid, 0.f);
        if constexpr (MASKED) {
            stm.store_strided(reinterpret_cast<uint32_t*>(sc + 3), 4, crow);
            stm.store(reinterpret_cast<uint32_t*>(oyd + crow * R * 2), crow);   // flags for the flush
        }
        __syncthreads();
        if (wrow0 == 0) {                                     // tape capture: bit copies
            const size_t bt0 = static_cast<size_t>(b) * T + t0;
            const float* flags = MASKED ? sc + 3 : nullptr;
            if (k_log != nullptr)
                stk.store_global(static_cast<char*>(k_log) + ((bt0 * Hv + hv) * DK) * EB,
                                 static_cast<size_t>(Hv) * DK, valid, flags);
            if (g_log != nullptr)
                stg.store_global(static_cast<char*>(g_log) + (bt0 * Hv + hv) * EB, Hv, valid, flags);
        }
        // k . q of each step: one 16-lane row group per step
        for (int tt = static_cast<int>(slot); tt < valid; tt += SLOTS) {
            float tk[E], tq[E];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float a[W], bq[W];
                lds_load_vec<W>(sk + tt * DK + (c * L + lane) * W, a);
                lds_load_vec<W>(sq + tt * DK + (c * L + lane) * W, bq);
#pragma unroll
                for (int w = 0; w < W; ++w) { tk[c * W + w] = a[w]; tq[c * W + w] = bq[w]; }
            }
            float kqs[1] = {lane_dot<E>(tk, tq)};
            row16_sum_n<1>(kqs);
            if (lane == 0) sc[4 * tt + 2] = kqs[0];
        }
        for (int tt = valid + static_cast<int>(threadIdx.x); tt < crow; tt += NT) sc[4 * tt + 2] = 0.f;
        __syncthreads();
        if (t0 + TC < T) load_chunk(t0 + TC);                 // in flight during this chunk
        if (t0 != 0) flush_chunk(t0 - TC);                    // the other output buffer

        // Steps in groups of kGroup: the group's LDS reads are issued together
        // (straight-line code, so each step waits only for its own operands),
        // then its steps run.  Rows past the tape end are padding with mask 0.
        auto run = [&](const StepOperands<E, RPT>& op, int tt) {
            if constexpr (MASKED) {
                if (__builtin_amdgcn_readfirstlane(__float_as_uint(op.sc.w)) == 0u) return;   // inactive
            }
            float d[RPT], out[RPT];
            record_step<RPT, E>(s, op.k, op.q, op.v, op.sc.x, op.sc.y, op.sc.z, d, out);
            float pair[2 * RPT];                              // all 16 lanes hold the same values
#pragma unroll
            for (int r = 0; r < RPT; ++r) { pair[2 * r] = out[r]; pair[2 * r + 1] = d[r]; }
            lds_store_vec<2 * RPT>(oyd + (tt * R + slot * RPT) * 2, pair);
        };
        StepOperands<E, RPT> op[G];
        for (int t4 = 0; t4 < valid; t4 += G) {
#pragma unroll
            for (int u = 0; u < G; ++u) op[u].template read<DK, R>(sk, sq, sv, sc, t4 + u, lane, slot);
#pragma unroll
            for (int u = 0; u < G; ++u) run(op[u], t4 + u);
        }
    }
    __syncthreads();
    flush_chunk(((T - 1) / TC) * TC);

    store_state_rows<RPT, E>(state_out + srow, lane, s);
}

template <int IO, int DK, int RPT, int NT>
hipError_t launch_cfg(const RecordArgs& a, hipStream_t stream) {
    constexpr int R = RPT * NT / 16;
    const uint32_t row_blocks = a.Dv / R;
    const uint64_t grid = static_cast<uint64_t>(a.B) * a.Hv * row_blocks;
    if (a.T == 1) {
        hipLaunchKernelGGL((gdn_record_kernel<IO, DK, RPT, NT>), dim3(static_cast<uint32_t>(grid)),
                           dim3(NT), 0, stream, a.q, a.k, a.v, a.g, a.beta, a.state_in, a.mask, a.y,
                           a.state_out, a.delta_log, a.k_log, a.g_log, a.Hk, a.Hv, a.Dv,
                           row_blocks, a.map);
        return hipGetLastError();
    }
    if constexpr (RPT <= 2) {
        if (a.T <= kShortDirectSteps) {
            hipLaunchKernelGGL((gdn_record_short_kernel<IO, DK, RPT, NT, kShortDirectSteps>),
                               dim3(static_cast<uint32_t>(grid)), dim3(NT), 0, stream, a.q, a.k, a.v, a.g,
                               a.beta, a.state_in, a.mask, a.y, a.state_out, a.delta_log, a.k_log, a.g_log,
                               a.T, a.Hk, a.Hv, a.Dv, row_blocks, a.map);
            return hipGetLastError();
        }
    }
    if constexpr (R <= kStagedMaxRows) {
        const bool masked = a.mask != nullptr;
        auto go = [&](auto kernel_masked, auto kernel_plain, uint32_t crow) {
            const size_t lds = record_lds_floats(static_cast<int>(crow), DK, R) * sizeof(float);
            hipLaunchKernelGGL(masked ? kernel_masked : kernel_plain, dim3(static_cast<uint32_t>(grid)),
                               dim3(NT), lds, stream, a.q, a.k, a.v, a.g, a.beta, a.state_in, a.mask,
                               a.y, a.state_out, a.delta_log, a.k_log, a.g_log, a.T, a.Hk, a.Hv, a.Dv,
                               row_blocks, a.map, crow);
        };
        if (a.T <= kShortChunk) {
            go(gdn_record_staged_kernel<IO, DK, RPT, NT, true, kShortChunk>,
               gdn_record_staged_kernel<IO, DK, RPT, NT, false, kShortChunk>, a.T);
        } else if (a.T <= static_cast<uint32_t>(kMediumChunk) || staged_chunk<DK>() <= kMediumChunk) {
            go(gdn_record_staged_kernel<IO, DK, RPT, NT, true, kMediumChunk>,
               gdn_record_staged_kernel<IO, DK, RPT, NT, false, kMediumChunk>,
               chunk_alloc_rows(kMediumChunk, a.T));
        } else {
            constexpr int TC = staged_chunk<DK>();
            if constexpr (RPT == 1 && DK <= 128) {
                if (grid <= compute_units()) {
                    go(gdn_record_staged_kernel<IO, DK, RPT, NT, true, kWideChunk>,
                       gdn_record_staged_kernel<IO, DK, RPT, NT, false, kWideChunk>,
                       chunk_alloc_rows(kWideChunk, a.T));
                    return hipGetLastError();
                }
            }
            go(gdn_record_staged_kernel<IO, DK, RPT, NT, true, TC>,
               gdn_record_staged_kernel<IO, DK, RPT, NT, false, TC>, chunk_alloc_rows(TC, a.T));
        }
        return hipGetLastError();
    }
    return hipErrorInvalidConfiguration;         // record_tiling never picks this for T > 1
}

template <int IO, int DK>
hipError_t launch_dk(const RecordArgs& a, const RowTiling& t, hipStream_t stream) {
    const int key = t.rows_per_thread * 1000 + t.threads;
    switch (key) {
        case 8256:
            if constexpr (8 * (DK / 16) <= kMaxStatePerLane) return launch_cfg<IO, DK, 8, 256>(a, stream);
            break;
        case 4256:
            if constexpr (4 * (DK / 16) <= kMaxStatePerLane) return launch_cfg<IO, DK, 4, 256>(a, stream);
            break;
        case 2256: return launch_cfg<IO, DK, 2, 256>(a, stream);
        case 1256: return launch_cfg<IO, DK, 1, 256>(a, stream);
        case 1064: return launch_cfg<IO, DK, 1, 64>(a, stream);
        default: break;
    }
    return hipErrorInvalidConfiguration;
}

template <int IO>
hipError_t launch_io(const RecordArgs& a, const RowTiling& t, hipStream_t stream) {
    switch (a.Dk) {
        case 32: return launch_dk<IO, 32>(a, t, stream);
        case 64: return launch_dk<IO, 64>(a, t, stream);
        case 128: return launch_dk<IO, 128>(a, t, stream);
        case 192: return launch_dk<IO, 192>(a, t, stream);
        case 256: return launch_dk<IO, 256>(a, t, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Compute units of the current device (cached per device; 256, the MI355X
// count, if the runtime cannot say).
uint32_t compute_units() {
    constexpr int kDevices = 64;
    static std::atomic<uint32_t> cache[kDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 256;
    uint32_t c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        c = static_cast<uint32_t>(n);
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

bool dk_supported(uint32_t Dk) {
    return Dk == 32 || Dk == 64 || Dk == 128 || Dk == 192 || Dk == 256;
}

RowTiling record_tiling(const RecordArgs& a) {
    if (a.forced.rows_per_thread != 0) return a.forced;      // checked by the caller
    // Up to 16 steps (speculative decode, and decode at Dk below 128): two
    // rows per thread over 256-thread groups measured fastest while that still
    // gives 1024 groups (20% faster than one row per thread at an 8-sequence
    // speculative step, where each thread's two rows keep twice the loads in
    // flight); then one row per thread, then one-wave groups.  Long tapes take
    // 16-row groups (one per CU at a 32-head prefill), or one-wave groups when
    // even that leaves CUs idle.
    static const int kShort[] = {3, 4};             // (1,256), (1,64)
    static const int kLong[] = {3, 4};              // (1,256), (1,64)
    const uint64_t heads = static_cast<uint64_t>(a.B) * a.Hv;
    // One step at Dk >= 128: one row per thread (two 16-byte state pieces or
    // more per lane already), 352 against 357 us a decode step of 512 MiB
    // of state run back to back, every write-back paid.
    if (a.T == 1 && a.Dk >= 128) return pick_tiling(heads, a.Dk, a.Dv, 2048, kShort, 2);
    if (a.T <= 16) {
        const RowTiling& wide = kTilings[2];                  // (2,256)
        if (tiling_fits(wide, a.Dk, a.Dv) && heads * (a.Dv / wide.rows()) >= 1024) return wide;
        return pick_tiling(heads, a.Dk, a.Dv, 2048, kShort, 2);
    }
    return pick_tiling(heads, a.Dk, a.Dv, 256, kLong, 2);
}

hipError_t launch_record(const RecordArgs& a, hipStream_t stream) {
    if (record_mfma_applies(a)) return launch_record_mfma(a, stream);
    const RowTiling t = record_tiling(a);
    switch (a.io) {
        case kF32: return launch_io<kF32>(a, t, stream);
        case kF16: return launch_io<kF16>(a, t, stream);
        case kBF16: return launch_io<kBF16>(a, t, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
