// gdn_replay: re-fold the accepted prefix of an innovation tape onto a
// pre-record state snapshot (speculative-decode rollback), gfx950.
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
// position: an untaken slot is never fetched (less tape traffic) and can never
// leak into the state, NaN or not.  The loop stops at min(accepted, T_log).
// The update is fma(k, delta, S * g): the same two roundings as the record
// kernel's decay followed by its rank-1 write, so replaying a full fp32 tape
// reproduces the record kernel's state bit for bit.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

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

    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const uint32_t rb = blk % row_blocks;
    const uint32_t n = blk / row_blocks;          // b * Hv + hv
    const uint32_t b = n / Hv;
    const uint32_t hv = n - b * Hv;

    const uint32_t row0 = rb * R + slot * RPT;
    const size_t srow = (static_cast<size_t>(n) * Dv + row0) * DK;

    float s[RPT][E];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float t4[W];
            f32_load_vec<W>(state_in + srow + r * DK + (c * L + lane) * W, t4);
#pragma unroll
            for (int w = 0; w < W; ++w) s[r][c * W + w] = t4[w];
        }

    for (uint32_t t = 0; t < steps; ++t) {
        const size_t bt = static_cast<size_t>(b) * T_log + t;
        if (mask != nullptr && mask[bt] == 0u) continue;     // untaken position

        const size_t gi = bt * Hv + hv;
        const float gt = io_load1<IO>(g_log, gi);
        float kk[E], dd[RPT];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float tk[W];
            io_load_vec<IO, W>(k_log, gi * DK + (c * L + lane) * W, tk);
#pragma unroll
            for (int w = 0; w < W; ++w) kk[c * W + w] = tk[w];
        }
        io_load_vec<IO, RPT>(delta_log, gi * Dv + row0, dd);

#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) s[r][e] = fmaf(kk[e], dd[r], s[r][e] * gt);
    }

#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float t4[W];
#pragma unroll
            for (int w = 0; w < W; ++w) t4[w] = s[r][c * W + w];
            f32_store_vec_nt<W>(state_out + srow + r * DK + (c * L + lane) * W, t4);
        }
}

template <int IO, int DK, int RPT, int NT>
hipError_t launch_cfg(const ReplayArgs& a, hipStream_t stream) {
    constexpr int R = RPT * NT / 16;
    const uint32_t row_blocks = a.Dv / R;
    const uint64_t grid = static_cast<uint64_t>(a.B) * a.Hv * row_blocks;
    hipLaunchKernelGGL((gdn_replay_kernel<IO, DK, RPT, NT>), dim3(static_cast<uint32_t>(grid)),
                       dim3(NT), 0, stream, a.delta_log, a.k_log, a.g_log, a.state_in, a.mask,
                       a.state_out, a.T_log, a.Hv, a.Dv, row_blocks, a.steps);
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
    RowTiling t;
    if (tiling_override("GDN_REPLAY_TILING", a.Dk, a.Dv, &t)) return t;
    return pick_tiling(static_cast<uint64_t>(a.B) * a.Hv, a.Dk, a.Dv, 2048);
}

hipError_t launch_replay(const ReplayArgs& a, hipStream_t stream) {
    const RowTiling t = replay_tiling(a);
    switch (a.io) {
        case kF32: return launch_io<kF32>(a, t, stream);
        case kF16: return launch_io<kF16>(a, t, stream);
        case kBF16: return launch_io<kBF16>(a, t, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
