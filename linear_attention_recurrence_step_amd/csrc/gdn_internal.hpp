// Host-side interface between the C ABI (gdn_abi.cpp) and the kernel launchers
// (gdn_record.hip, gdn_replay.hip, gqa_expand.hip).  Arguments arrive here
// already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Row blocking of a head: a workgroup of `threads` threads covers
// rows_per_thread * threads / 16 consecutive value rows of one head.
// rows_per_thread == 0 stands for "not forced" in the argument structs.
struct RowTiling {
    int rows_per_thread;
    int threads;
    int rows() const { return rows_per_thread * threads / 16; }
};

// Which kernel folds a replay (same values as gdn_replay_fold in gdn.h).
enum ReplayFold : int { kFoldAuto = 0, kFoldValu = 1, kFoldMatrix = 2 };

struct RecordArgs {
    const void* q; const void* k; const void* v; const void* g; const void* beta;
    const float* state_in; const uint32_t* mask;
    void* y; float* state_out; void* delta_log;
    void* k_log; void* g_log;             // optional tape capture
    uint32_t B, T, Hk, Hv, Dk, Dv;
    int io;       // IoType
    int map;      // 0 block, 1 tiled
    RowTiling forced;                     // {0, 0}: the launcher picks
};

struct ReplayArgs {
    const void* delta_log; const void* k_log; const void* g_log;
    const float* state_in; const uint32_t* mask; float* state_out;
    uint32_t B, T_log, Hv, Dk, Dv, steps;   // steps = min(accepted, T_log)
    int io;
    RowTiling forced;                     // VALU folds; {0, 0}: the launcher picks
    int fold;                             // ReplayFold
    uint32_t matrix_waves;                // matrix-core fold: 2 or 4 waves; 0: the launcher picks
};

struct ExpandArgs {
    const void* src; void* dst;
    uint32_t seq, hg, h, k;
    uint32_t elem_bytes;
    int map;
};

// Does a kernel exist for this key width?
bool dk_supported(uint32_t Dk);

// Compute units of the current device (cached per device; 256, the MI355X
// count, if the runtime cannot say).
uint32_t compute_units();

// Tiling the launchers will use (also used by the ABI for its grid-size check).
RowTiling record_tiling(const RecordArgs& a);
RowTiling replay_tiling(const ReplayArgs& a);

hipError_t launch_record(const RecordArgs& a, hipStream_t stream);

// Records of 2..4 steps of bf16 I/O with Dk in {32, 64, 128, 192} and Dv a
// multiple of 16 (and no forced tiling) run their dense products on the
// matrix cores (gdn_record_mfma.hip, one 16-row wave per workgroup).
bool record_mfma_applies(const RecordArgs& a);
hipError_t launch_record_mfma(const RecordArgs& a, hipStream_t stream);
hipError_t launch_replay(const ReplayArgs& a, hipStream_t stream);

struct RmsNormArgs {
    const float* x; const uint16_t* weight; float* out;
    uint32_t n_tokens, dim;
    float eps;
};
hipError_t launch_rms_norm(const RmsNormArgs& a, hipStream_t stream);

// Folds of at least this many positions of a 16-bit tape run as matrix
// products on the matrix cores (gdn_replay_mfma.hip).
inline constexpr uint32_t kReplayMfmaFromSteps = 16;
// Whether the matrix-core fold can take this replay at all (16-bit tape,
// whole 64-row workgroups, grid within one launch), and whether the launcher
// sends it there (that, and the fold chosen or the length rule above).
bool replay_mfma_possible(const ReplayArgs& a);
bool replay_mfma_applies(const ReplayArgs& a);
hipError_t launch_replay_mfma(const ReplayArgs& a, hipStream_t stream);
hipError_t launch_expand(const ExpandArgs& a, hipStream_t stream);

// Chunked prefill (gdn_prefill.hip): the record step computed 64 steps at a
// time on the matrix cores, through a caller-provided workspace.
struct PrefillArgs {
    const void* q; const void* k; const void* v; const void* g; const void* beta;
    const float* state_in; const uint32_t* mask;
    void* y; float* state_out; void* delta_log;
    void* k_log; void* g_log;             // optional tape capture
    void* workspace;
    uint32_t B, T, Hk, Hv, Dk, Dv;
    int io;
    int map;      // 0 block, 1 tiled
};
uint64_t prefill_workspace_bytes(uint32_t B, uint32_t T, uint32_t Hv);   // UINT64_MAX if it overflows
bool prefill_supported(uint32_t Dk, uint32_t Dv, int io);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// The allocation-free prefill's workspace: a file-scope device array of this
// many bytes in gdn_prefill.hip (2048 blocks of 33280 bytes: a 4096-step
// prefill over 32 value heads).  prefill_scratch() gives its address on the
// device `stream` runs on, looked up once per device; that device must be
// the current one (hipErrorInvalidDevice otherwise).
inline constexpr uint64_t kPrefillScratchBytes = 68157440ull;
hipError_t prefill_scratch(hipStream_t stream, void** out);

}  // namespace gdn

namespace gdn {

// Candidate row tilings, widest first.  A lane keeps rows_per_thread * Dk / 16
// state values in registers; that is held to at most 64.
inline constexpr RowTiling kTilings[] = {{8, 256}, {4, 256}, {2, 256}, {1, 256}, {1, 64}};
inline constexpr int kNumTilings = 5;
inline constexpr int kMaxStatePerLane = 64;

inline bool tiling_fits(const RowTiling& t, uint32_t Dk, uint32_t Dv) {
    return Dv % static_cast<uint32_t>(t.rows()) == 0 &&
           static_cast<uint32_t>(t.rows_per_thread) * (Dk / 16) <= kMaxStatePerLane;
}

// First tiling of `prefs` (a list of kTilings indices) that fits and still
// yields `target_groups` workgroups; otherwise the narrowest tiling that fits
// (more, smaller workgroups for few heads).
inline RowTiling pick_tiling(uint64_t heads, uint32_t Dk, uint32_t Dv, uint64_t target_groups,
                             const int* prefs, int nprefs) {
    for (int i = 0; i < nprefs; ++i) {
        const RowTiling& t = kTilings[prefs[i]];
        if (tiling_fits(t, Dk, Dv) && heads * (Dv / t.rows()) >= target_groups) return t;
    }
    for (int i = kNumTilings - 1; i >= 0; --i)
        if (tiling_fits(kTilings[i], Dk, Dv)) return kTilings[i];
    return kTilings[kNumTilings - 1];
}

// Largest row block (rows per workgroup) the staged record kernel takes; it
// bounds that kernel's LDS below 64 KiB.
inline constexpr int kStagedMaxRows = 64;

// Whether (rows_per_thread, threads) is one of kTilings.
inline bool tiling_known(int rows_per_thread, int threads) {
    for (int i = 0; i < kNumTilings; ++i)
        if (kTilings[i].rows_per_thread == rows_per_thread && kTilings[i].threads == threads) return true;
    return false;
}

}  // namespace gdn
