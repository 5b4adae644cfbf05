// gdn_replay: the speculative-decode rollback on gfx950 -- from the state saved
// before the record, apply the accepted positions of the innovation tape.
//
// What it computes is the replay kernel (macro `state_replay!`) of the
// metaltile-std 0.1.0 page src/ffai/gated_delta_replay.rs: per (b, hv, dv) row,
// for each tape position t < accepted whose mask entry passes,
//     S[dv,:] <- S[dv,:] * g_log[t] + k_log[t,:] * delta_log[t,dv],
// and nothing for any other position.
//
// Mapping (same row tiling as gdn_record): 16 lanes share a row, a thread owns
// RPT consecutive rows held in VGPRs, the snapshot is read once and the result
// written once.  The page expresses "skip this position" as a per-lane select
// between new and old state.  Here the step flag depends only on (b, t), which
// is uniform over a workgroup, so it becomes a scalar branch around the whole
// position: an untaken slot can never leak into the state, NaN or not.  The
// loop stops at min(accepted, T_log), so positions past it are never fetched.
// The update is fma(k, delta, S * g): the same two roundings as the record
// kernel's decay followed by its rank-1 write, so replaying a full fp32 tape
// reproduces the record kernel's state bit for bit.  A fold of one position
// runs the direct kernel below; longer folds run the staged kernel, which
// brings the tape in through LDS a chunk of positions at a time.  Folds of 16
// or more positions carry the state as scale * s (S = g S + delta k^T becomes
// scale *= g, s += (delta / scale) k), which halves the arithmetic per
// position; the result equals the direct fold up to rounding.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

// At most one taken position (steps <= 1, so only position 0 can be taken):
// the state loads and position 0's tape loads go out together, the fold
// runs at most once, and there is no position loop (its loop-carried state
// registers had made the compiler wait for the state before issuing the
// tape's loads).
template <int IO, int DK, int RPT, int NT>
__global__ __launch_bounds__(NT) void gdn_replay_kernel(
    const void* __restrict__ delta_log, const void* __restrict__ k_log,
    const void* __restrict__ g_log, const float* state_in,
    const uint32_t* __restrict__ mask, float* state_out,
    uint32_t T_log, uint32_t Hv, uint32_t Dv, uint32_t row_blocks, uint32_t steps)
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

    // Rows [blk*R, blk*R + R) of the flattened [B*Hv*Dv] row space; the state
    // address needs no division, so its loads are issued first.
    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const size_t srow = (static_cast<size_t>(blk) * R + slot * RPT) * DK;

    float s[RPT][E];
    load_state_rows<RPT, E>(state_in + srow, lane, s);

    const uint32_t n = blk / row_blocks;          // b * Hv + hv
    const uint32_t row0 = (blk - n * row_blocks) * R + slot * RPT;
    const uint32_t b = n / Hv;
    const uint32_t hv = n - b * Hv;
    const size_t bt = static_cast<size_t>(b) * T_log;         // position 0
    const size_t gi = bt * Hv + hv;

    RawIo<IO, W> kr[NC];
    RawIo<IO, RPT> dr;
    RawIo<IO, 1> gr;
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c].load(k_log, gi * DK + (c * L + lane) * W);
    dr.load(delta_log, gi * Dv + row0);
    gr.load(g_log, gi);
    const bool take = steps > 0u && (mask == nullptr || mask[bt] != 0u);

    if (take) {
        const float gt = gr.at(0);
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float dd = dr.at(r);
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int w = 0; w < W; ++w)
                    s[r][c * W + w] = fmaf(kr[c].at(w), dd, s[r][c * W + w] * gt);
        }
    }

    store_state_rows<RPT, E>(state_out + srow, lane, s);
}

// The LDS operands of one tape position for one lane: its E columns of k_log,
// the delta values of its RPT rows, the gate and the mask entry.
template <int E, int RPT, int R>
struct TapeOperands {
    float k[E], d[RPT], g;
    uint32_t m;
    __device__ __forceinline__ void read(const float* sk, const float* sd, const float* sg,
                                         const uint32_t* sm, int tt, uint32_t lane, uint32_t slot) {
        constexpr int L = 16;
        constexpr int W = E < 4 ? E : 4;
        constexpr int DK = E * L;
#pragma unroll
        for (int c = 0; c < E / W; ++c) {
            float tk[W];
            lds_load_vec<W>(sk + tt * DK + (c * L + lane) * W, tk);
#pragma unroll
            for (int w = 0; w < W; ++w) k[c * W + w] = tk[w];
        }
        lds_load_vec<RPT>(sd + tt * R + slot * RPT, d);
        g = sg[tt];
        m = sm[tt];
    }
};

template <int DK>
constexpr int replay_chunk() { return DK <= 128 ? 32 : 16; }

// Positions whose LDS operands are read together; LDS chunks are padded to a
// multiple of this many rows.
constexpr int kGroup = 4;

// Whether c0 times every prefix product of the taken gates of a chunk (up to
// 32 positions, from LDS) stays within [2^-64, 2^64], so that a scaled fold
// of the chunk keeps a finite, well-scaled 1 / scale.  Lane i of each wave
// takes position i; a log-step prefix product and a ballot make the answer
// uniform.  NaN or infinite gates fail the test.
__device__ __forceinline__ bool scale_stays_in_range(const float* sg, const uint32_t* sm,
                                                     int valid, float c0) {
    const int i = static_cast<int>(threadIdx.x & 31u);
    float f = (i < valid && sm[i] != 0u) ? sg[i] : 1.f;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
        const float o = __shfl_up(f, off, 32);
        if (i >= off) f *= o;
    }
    const uint32_t mag = __float_as_uint(f * c0) & 0x7fffffffu;
    const bool bad = i < valid && !(mag >= 0x1f800000u && mag <= 0x5f800000u);
    return (__ballot(bad) & 0xffffffffull) == 0ull;
}

// Folds of at least this many positions carry the state with a running scale
// (one FMA per value and position); shorter folds use the direct update,
// which reproduces the record kernel's roundings exactly.
constexpr uint32_t kScaledFromSteps = 16;

// LDS floats for a chunk of `rows` positions: k_log rows, this group's delta, g, mask.
__host__ __device__ constexpr size_t replay_lds_floats(int rows, int dk, int r) {
    return static_cast<size_t>(rows) * (dk + r + 2);
}

// Staged variant for more than one position: the tape data of a chunk of TC
// positions (the k_log row and g of this head, delta of this group's rows, the
// mask entries) is copied into LDS as float32 in one round of coalesced loads,
// and the following chunk is loaded into registers while the current one is
// folded.  Positions whose mask entry is zero are skipped, never folded.
template <int IO, int DK, int RPT, int NT, bool SCALED>
__global__ __launch_bounds__(NT) void gdn_replay_staged_kernel(
    const void* __restrict__ delta_log, const void* __restrict__ k_log,
    const void* __restrict__ g_log, const float* state_in,
    const uint32_t* __restrict__ mask, float* state_out,
    uint32_t T_log, uint32_t Hv, uint32_t Dv, uint32_t row_blocks, uint32_t steps,
    uint32_t chunk_rows)
{
    constexpr int L = 16;
    constexpr int E = DK / L;
    constexpr int W = E < 4 ? E : 4;
    constexpr int NC = E / W;
    constexpr int SLOTS = NT / L;
    constexpr int R = SLOTS * RPT;
    constexpr int TC = replay_chunk<DK>();
    // positions whose operands are read together: with several rows per
    // thread one position's FMAs already cover an LDS read, and fewer
    // operand sets in flight keep the register count down
    constexpr int G = RPT >= 4 ? 1 : kGroup / RPT;
    constexpr int EB = IoTraits<IO>::kBytes;
    static_assert(DK % (L * W) == 0 && NC * W == E, "unsupported Dk");

    extern __shared__ __align__(16) float lds[];
    const int crow = static_cast<int>(chunk_rows);            // min(TC, steps) rounded up to kGroup
    float* sk = lds;
    float* sd = sk + crow * DK;
    float* sg = sd + crow * R;
    uint32_t* sm = reinterpret_cast<uint32_t*>(sg + crow);

    const uint32_t lane = threadIdx.x & (L - 1);
    const uint32_t slot = threadIdx.x / L;
    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const size_t srow = (static_cast<size_t>(blk) * R + slot * RPT) * DK;

    float s[RPT][E];
    load_state_rows<RPT, E>(state_in + srow, lane, s);

    const uint32_t n = blk / row_blocks;          // b * Hv + hv
    const uint32_t wrow0 = (blk - n * row_blocks) * R;
    const uint32_t b = n / Hv;
    const uint32_t hv = n - b * Hv;

    ChunkStager<IO, TC, DK, piece_elems<IO, DK>(), NT> stk;
    ChunkStager<IO, TC, R, piece_elems<IO, R>(), NT> std_;
    ChunkStager<IO, TC, 1, 1, NT> stg;
    MaskStager<TC, NT> stm;

    auto load_chunk = [&](uint32_t t0) {
        const int valid = static_cast<int>(steps - t0 < TC ? steps - t0 : TC);
        const size_t bt0 = static_cast<size_t>(b) * T_log + t0;
        stk.load(static_cast<const char*>(k_log) + ((bt0 * Hv + hv) * DK) * EB,
                 static_cast<size_t>(Hv) * DK, valid);
        std_.load(static_cast<const char*>(delta_log) + ((bt0 * Hv + hv) * Dv + wrow0) * EB,
                  static_cast<size_t>(Hv) * Dv, valid);
        stg.load(static_cast<const char*>(g_log) + (bt0 * Hv + hv) * EB, Hv, valid);
        stm.load(mask != nullptr ? mask + bt0 : nullptr, valid);
    };

    // SCALED: the state is carried as scale * s with a workgroup-uniform
    // scale (the gate is per head), so a taken position costs one FMA per
    // state value instead of a multiply and an FMA.
    float scale = 1.f;
    if (steps > 0) load_chunk(0);
    wait_vector_memory();                                     // snapshot rows and chunk 0 are in
    for (uint32_t t0 = 0; t0 < steps; t0 += TC) {
        if (t0 != 0) __syncthreads();
        stk.store(sk, crow);
        std_.store(sd, crow);
        stg.store(sg, crow);
        stm.store(sm, crow);
        __syncthreads();
        if (t0 + TC < steps) load_chunk(t0 + TC);
        const int valid = static_cast<int>(steps - t0 < TC ? steps - t0 : TC);

        // Positions in groups of kGroup: the group's LDS reads are issued
        // together (straight-line code, so each fold waits only for its own
        // operands), then the positions are folded in order.  Rows past the
        // end of the fold are padding with mask 0.
        TapeOperands<E, RPT, R> op[G];
        auto fold_direct = [&](const TapeOperands<E, RPT, R>& op) {
            if (__builtin_amdgcn_readfirstlane(op.m) == 0u) return;      // untaken position
            const float gt = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(op.g)));
#pragma unroll
            for (int r = 0; r < RPT; ++r)
#pragma unroll
                for (int e = 0; e < E; ++e) s[r][e] = fmaf(op.k[e], op.d[r], s[r][e] * gt);
        };
        // S = scale * s: a taken position does scale *= g, s += (delta / scale) k.
        auto fold_scaled = [&](const TapeOperands<E, RPT, R>& op) {
            if (__builtin_amdgcn_readfirstlane(op.m) == 0u) return;      // untaken position
            const float gt = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(op.g)));
            scale *= gt;
            const float inv = __builtin_amdgcn_rcpf(scale);
            float dd[RPT];
#pragma unroll
            for (int r = 0; r < RPT; ++r) dd[r] = op.d[r] * inv;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
#pragma unroll
                for (int e = 0; e < E; ++e) s[r][e] = fmaf(op.k[e], dd[r], s[r][e]);
        };
        bool scaled_chunk = false;
        if constexpr (SCALED) {
            scaled_chunk = scale_stays_in_range(sg, sm, valid, scale);
            if (!scaled_chunk) {
                // fold the scale into the state, then try again from 1
                if (scale != 1.f) {
#pragma unroll
                    for (int r = 0; r < RPT; ++r)
#pragma unroll
                        for (int e = 0; e < E; ++e) s[r][e] *= scale;
                    scale = 1.f;
                }
                scaled_chunk = scale_stays_in_range(sg, sm, valid, 1.f);
            }
        }
        if (scaled_chunk) {
            for (int t4 = 0; t4 < valid; t4 += G) {
#pragma unroll
                for (int u = 0; u < G; ++u) op[u].read(sk, sd, sg, sm, t4 + u, lane, slot);
#pragma unroll
                for (int u = 0; u < G; ++u) fold_scaled(op[u]);
            }
        } else {
            for (int t4 = 0; t4 < valid; t4 += G) {
#pragma unroll
                for (int u = 0; u < G; ++u) op[u].read(sk, sd, sg, sm, t4 + u, lane, slot);
#pragma unroll
                for (int u = 0; u < G; ++u) fold_direct(op[u]);
            }
        }
    }
    if (SCALED && scale != 1.f) {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) s[r][e] *= scale;
    }

    store_state_rows<RPT, E>(state_out + srow, lane, s);
}

template <int IO, int DK, int RPT, int NT>
hipError_t launch_cfg(const ReplayArgs& a, hipStream_t stream) {
    constexpr int R = RPT * NT / 16;
    const uint32_t row_blocks = a.Dv / R;
    const uint64_t grid = static_cast<uint64_t>(a.B) * a.Hv * row_blocks;
    if (a.steps <= 1) {
        hipLaunchKernelGGL((gdn_replay_kernel<IO, DK, RPT, NT>), dim3(static_cast<uint32_t>(grid)),
                           dim3(NT), 0, stream, a.delta_log, a.k_log, a.g_log, a.state_in, a.mask,
                           a.state_out, a.T_log, a.Hv, a.Dv, row_blocks, a.steps);
    } else {
        constexpr int TC = replay_chunk<DK>();
        const uint32_t crow = ((a.steps < static_cast<uint32_t>(TC) ? a.steps : TC) + kGroup - 1) / kGroup * kGroup;
        const size_t lds = replay_lds_floats(static_cast<int>(crow), DK, R) * sizeof(float);
        if (a.steps >= kScaledFromSteps)
            hipLaunchKernelGGL((gdn_replay_staged_kernel<IO, DK, RPT, NT, true>),
                               dim3(static_cast<uint32_t>(grid)), dim3(NT), lds, stream, a.delta_log,
                               a.k_log, a.g_log, a.state_in, a.mask, a.state_out, a.T_log, a.Hv, a.Dv,
                               row_blocks, a.steps, crow);
        else
            hipLaunchKernelGGL((gdn_replay_staged_kernel<IO, DK, RPT, NT, false>),
                               dim3(static_cast<uint32_t>(grid)), dim3(NT), lds, stream, a.delta_log,
                               a.k_log, a.g_log, a.state_in, a.mask, a.state_out, a.T_log, a.Hv, a.Dv,
                               row_blocks, a.steps, crow);
    }
    return hipGetLastError();
}

template <int IO, int DK>
hipError_t launch_dk(const ReplayArgs& a, const RowTiling& t, hipStream_t stream) {
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
hipError_t launch_io(const ReplayArgs& a, const RowTiling& t, hipStream_t stream) {
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

RowTiling replay_tiling(const ReplayArgs& a) {
    if (a.forced.rows_per_thread != 0) return a.forced;      // checked by the caller
    // One or two taken positions: a pure state stream, fastest with one row
    // per thread.  Longer folds share each position's tape data over more
    // rows per workgroup; four rows per thread measured fastest (eight cost
    // too many registers).
    static const int kShort[] = {3, 4, 2};          // (1,256), (1,64), (2,256)
    static const int kLong[] = {1, 2, 0, 3, 4};     // (4,256), (2,256), (8,256), ...
    const uint64_t heads = static_cast<uint64_t>(a.B) * a.Hv;
    if (a.steps <= 2) return pick_tiling(heads, a.Dk, a.Dv, 2048, kShort, 3);
    return pick_tiling(heads, a.Dk, a.Dv, 2048, kLong, 5);
}

hipError_t launch_replay(const ReplayArgs& a, hipStream_t stream) {
    if (replay_mfma_applies(a)) return launch_replay_mfma(a, stream);
    const RowTiling t = replay_tiling(a);
    switch (a.io) {
        case kF32: return launch_io<kF32>(a, t, stream);
        case kF16: return launch_io<kF16>(a, t, stream);
        case kBF16: return launch_io<kBF16>(a, t, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
