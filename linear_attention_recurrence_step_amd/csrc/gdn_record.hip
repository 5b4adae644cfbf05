// gdn_record: gated delta-rule forward step with innovation-tape capture, gfx950.
//
// What it computes is the record kernel (macro `gated_delta_record!`) of the
// metaltile-std 0.1.0 page src/ffai/gated_delta_replay.rs: per (b, hv, dv) row
// and active step t, decay the row by g, read it out against k, form the
// innovation delta = (v - kv) * beta, write delta to the tape, add delta * k to
// the row and read the row out against q into y.
//
// How it maps onto CDNA4 (not the page's one-32-lane-group-per-row layout):
//  * 16 lanes (one DPP row) share a state row; lane l holds the Dk/16 columns
//    {(c*16 + l)*W + w}, so every 16-lane vector access is contiguous.
//  * A thread owns RPT consecutive rows of one head; a workgroup of NT threads
//    covers RPT*NT/16 rows.  The rows stay in VGPRs for all T steps; the state
//    is read once and written once (non-temporal) per launch.
//  * Both Dk-length dot products finish with a 4-stage DPP butterfly inside the
//    16-lane row, so no LDS and no barrier is involved.
//  * k and q of a step are loaded per lane straight from global memory: the
//    16 column slices of one key head are shared by every row of the
//    workgroup, so the repeats hit the L1/L2, and HBM sees each key vector once
//    per XCD.
//  * The mask row [B, T] is uniform over a workgroup, so inactive steps are a
//    scalar branch around the whole step.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

#include <cstdlib>
#include <cstdio>

namespace gdn {
namespace {

template <int IO, int DK, int RPT, int NT>
__global__ __launch_bounds__(NT) void gdn_record_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ g, const void* __restrict__ beta,
    const float* state_in, const uint32_t* __restrict__ mask,
    void* __restrict__ y, float* state_out, void* __restrict__ delta_log,
    uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dv, uint32_t row_blocks, int tiled)
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

    // Logical work index: (b, key head, value head within the key head's
    // group, row block), so the groups sharing a key head sit next to each other.
    const uint32_t blk = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const uint32_t rb = blk % row_blocks;
    const uint32_t n = blk / row_blocks;
    const uint32_t b = n / Hv;
    const uint32_t m = n - b * Hv;
    const uint32_t group = Hv / Hk;
    const uint32_t hk = m / group;
    const uint32_t j = m - hk * group;
    const uint32_t hv = tiled ? j * Hk + hk : m;

    const uint32_t row0 = rb * R + slot * RPT;               // first row of this thread
    const size_t head = static_cast<size_t>(b) * Hv + hv;
    const size_t srow = (head * Dv + row0) * DK;

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

    for (uint32_t t = 0; t < T; ++t) {
        const size_t bt = static_cast<size_t>(b) * T + t;
        if (mask != nullptr && mask[bt] == 0u) continue;      // inactive step: no decay, no writes

        const size_t gi = bt * Hv + hv;
        const float gt = io_load1<IO>(g, gi);
        const float bt_beta = io_load1<IO>(beta, gi);
        const size_t kq = (bt * Hk + hk) * DK;
        const size_t vo = gi * Dv + row0;

        float kk[E], qq[E], vv[RPT];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float tk[W], tq[W];
            io_load_vec<IO, W>(k, kq + (c * L + lane) * W, tk);
            io_load_vec<IO, W>(q, kq + (c * L + lane) * W, tq);
#pragma unroll
            for (int w = 0; w < W; ++w) { kk[c * W + w] = tk[w]; qq[c * W + w] = tq[w]; }
        }
        io_load_vec<IO, RPT>(v, vo, vv);

        // decay, then read the decayed row out against k
        float kv[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                s[r][e] = s[r][e] * gt;
                acc = fmaf(s[r][e], kk[e], acc);
            }
            kv[r] = row16_sum(acc);
        }

        float d[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) d[r] = (vv[r] - kv[r]) * bt_beta;
        if (delta_log != nullptr && lane == 0) io_store_vec<IO, RPT>(delta_log, vo, d);

        // rank-1 write, then read the updated row out against q
        float out[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                s[r][e] = fmaf(kk[e], d[r], s[r][e]);
                acc = fmaf(s[r][e], qq[e], acc);
            }
            out[r] = row16_sum(acc);
        }
        if (lane == 0) io_store_vec<IO, RPT>(y, vo, out);
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
hipError_t launch_cfg(const RecordArgs& a, hipStream_t stream) {
    constexpr int R = RPT * NT / 16;
    const uint32_t row_blocks = a.Dv / R;
    const uint64_t grid = static_cast<uint64_t>(a.B) * a.Hv * row_blocks;
    hipLaunchKernelGGL((gdn_record_kernel<IO, DK, RPT, NT>), dim3(static_cast<uint32_t>(grid)),
                       dim3(NT), 0, stream, a.q, a.k, a.v, a.g, a.beta, a.state_in, a.mask, a.y,
                       a.state_out, a.delta_log, a.T, a.Hk, a.Hv, a.Dv, row_blocks, a.map);
    return hipGetLastError();
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

bool dk_supported(uint32_t Dk) {
    return Dk == 32 || Dk == 64 || Dk == 128 || Dk == 192 || Dk == 256;
}

bool tiling_override(const char* env_name, uint32_t Dk, uint32_t Dv, RowTiling* out) {
    const char* s = std::getenv(env_name);
    if (s == nullptr || *s == '\0') return false;
    int rpt = 0, nt = 0;
    if (std::sscanf(s, "%d,%d", &rpt, &nt) != 2) return false;
    for (int i = 0; i < kNumTilings; ++i) {
        if (kTilings[i].rows_per_thread == rpt && kTilings[i].threads == nt &&
            tiling_fits(kTilings[i], Dk, Dv)) {
            *out = kTilings[i];
            return true;
        }
    }
    return false;
}

RowTiling record_tiling(const RecordArgs& a) {
    RowTiling t;
    if (tiling_override("GDN_RECORD_TILING", a.Dk, a.Dv, &t)) return t;
    // Short tapes stream the state: wide row blocks keep many bytes in flight.
    // Long tapes are a serial chain per row: spread the rows over more CUs.
    const uint64_t target = a.T <= 16 ? 2048 : 4096;
    return pick_tiling(static_cast<uint64_t>(a.B) * a.Hv, a.Dk, a.Dv, target);
}

hipError_t launch_record(const RecordArgs& a, hipStream_t stream) {
    const RowTiling t = record_tiling(a);
    switch (a.io) {
        case kF32: return launch_io<kF32>(a, t, stream);
        case kF16: return launch_io<kF16>(a, t, stream);
        case kBF16: return launch_io<kBF16>(a, t, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
