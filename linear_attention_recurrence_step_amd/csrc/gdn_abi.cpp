// extern "C" boundary of libgdn: argument validation (entirely on the host,
// before any HIP call) and dispatch to the kernel launchers.
//
// The validation rules follow `dispatch_repeat_tiled_f32` on the mlx-native
// 0.6.5 page mlx_native/ops/repeat_tiled.rs (zero dimensions, the head ratio,
// size overflow) and the dispatch invariants of the metaltile-std 0.1.0 page
// src/ffai/gated_delta_replay.rs (Dk a multiple of 32), extended with the
// checks a raw-pointer interface needs (NULL, alignment, overlap).
#include "gdn.h"
#include "gdn_internal.hpp"

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

// a * b * c * d * e in 64 bits; false on overflow.
bool mul_u64(uint64_t* out, std::initializer_list<uint64_t> xs) {
    uint64_t acc = 1;
    for (uint64_t x : xs)
        if (__builtin_mul_overflow(acc, x, &acc)) return false;
    *out = acc;
    return true;
}

constexpr uint64_t kMaxBytes = uint64_t(1) << 48;   // 256 TiB: far beyond any device, safe for offsets
// A launch covers at most 2^32 - 1 work-items (the dispatch packet's grid
// size is 32 bits wide).
constexpr uint64_t kMaxWorkItems = 0xffffffffull;

static_assert(GDN_PREFILL_SCRATCH_BYTES == gdn::kPrefillScratchBytes, "gdn.h and the library disagree");

struct Span {
    const void* p;
    uint64_t bytes;
    const char* name;
};

bool overlaps(const Span& a, const Span& b) {
    if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int io_bytes(int dtype) { return dtype == GDN_F32 ? 4 : 2; }

bool valid_dtype(int d) { return d == GDN_F32 || d == GDN_F16 || d == GDN_BF16; }
bool valid_map(int m) { return m == GDN_GQA_BLOCK || m == GDN_GQA_TILED; }

int launch_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return GDN_OK;
    return fail(GDN_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_last_error(void) { return g_last_error; }

const char* gdn_strerror(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_ZERO_DIM: return "a dimension is zero";
        case GDN_ERR_GQA_RATIO: return "the key-head count does not divide the value-head count";
        case GDN_ERR_UNSUPPORTED_SHAPE: return "unsupported head dimensions";
        case GDN_ERR_OVERFLOW: return "tensor size or launch grid too large";
        case GDN_ERR_ALIAS: return "an output overlaps an input or another output";
        case GDN_ERR_BAD_ENUM: return "unknown dtype or GQA map";
        case GDN_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
        case GDN_ERR_MISALIGNED: return "a pointer is not aligned as required";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// The tiling a launch choice forces ({0, 0}: none), after checking it against
// the shape; returns GDN_OK or the status to fail with (message set).
int forced_tiling(const gdn_launch_choice* c, const char* fn, uint32_t Dk, uint32_t Dv,
                  uint32_t max_rows, gdn::RowTiling* out) {
    *out = gdn::RowTiling{0, 0};
    if (c == nullptr || (c->rows_per_thread == 0 && c->threads == 0)) return GDN_OK;
    const int rpt = static_cast<int>(c->rows_per_thread), nt = static_cast<int>(c->threads);
    if (c->rows_per_thread > 8 || c->threads > 256 || !gdn::tiling_known(rpt, nt))
        return fail(GDN_ERR_BAD_ENUM, "%s: no row tiling of %u rows per thread over %u threads", fn,
                    c->rows_per_thread, c->threads);
    const gdn::RowTiling t{rpt, nt};
    if (!gdn::tiling_fits(t, Dk, Dv) || static_cast<uint32_t>(t.rows()) > max_rows)
        return fail(GDN_ERR_UNSUPPORTED_SHAPE,
                    "%s: a tiling of %d rows per thread over %d threads does not fit Dk=%u, Dv=%u "
                    "(at most %u rows per workgroup here)", fn, rpt, nt, Dk, Dv, max_rows);
    *out = t;
    return GDN_OK;
}

int record_impl(const gdn_launch_choice* choice,
                const void* q, const void* k, const void* v, const void* g, const void* beta,
                const float* state_in, const uint32_t* mask,
                void* y, float* state_out, void* delta_log, void* k_log, void* g_log,
                uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                int io_dtype, int gqa_map, void* stream, const char* kFn) {
    if (!valid_dtype(io_dtype)) return fail(GDN_ERR_BAD_ENUM, "%s: unknown io_dtype %d", kFn, io_dtype);
    if (!valid_map(gqa_map)) return fail(GDN_ERR_BAD_ENUM, "%s: unknown gqa_map %d", kFn, gqa_map);
    if (!q || !k || !v || !g || !beta || !state_in || !y || !state_out)
        return fail(GDN_ERR_NULL, "%s: one of q, k, v, g, beta, state_in, y, state_out is NULL", kFn);
    if (B == 0 || T == 0 || Hk == 0 || Hv == 0 || Dk == 0 || Dv == 0)
        return fail(GDN_ERR_ZERO_DIM, "%s: zero-sized dimension in B=%u T=%u Hk=%u Hv=%u Dk=%u Dv=%u",
                    kFn, B, T, Hk, Hv, Dk, Dv);
    if (Hv % Hk != 0)
        return fail(GDN_ERR_GQA_RATIO, "%s: %u value heads cannot share %u key heads evenly", kFn, Hv, Hk);
    if (!gdn::dk_supported(Dk) || Dv % 16 != 0 || Dv > 1024)
        return fail(GDN_ERR_UNSUPPORTED_SHAPE,
                    "%s: no kernel for Dk=%u, Dv=%u (Dk in {32, 64, 128, 192, 256}; Dv a multiple "
                    "of 16, at most 1024)", kFn, Dk, Dv);
    if (choice != nullptr && (choice->replay_fold != 0 || choice->matrix_waves != 0))
        return fail(GDN_ERR_BAD_ENUM, "%s: replay_fold and matrix_waves apply to the replay only", kFn);
    gdn::RowTiling forced;
    {
        const uint32_t max_rows = T == 1 ? 1024u : static_cast<uint32_t>(gdn::kStagedMaxRows);
        const int st = forced_tiling(choice, kFn, Dk, Dv, max_rows, &forced);
        if (st != GDN_OK) return st;
    }

    const uint64_t e = io_bytes(io_dtype);
    uint64_t n_qk, n_v, n_g, n_s, n_m, n_kl;
    if (!mul_u64(&n_qk, {B, T, Hk, Dk, e}) || !mul_u64(&n_v, {B, T, Hv, Dv, e}) ||
        !mul_u64(&n_g, {B, T, Hv, e}) || !mul_u64(&n_s, {B, Hv, Dv, Dk, 4}) || !mul_u64(&n_m, {B, T, 4}) ||
        !mul_u64(&n_kl, {B, T, Hv, Dk, e}) ||
        n_qk > kMaxBytes || n_v > kMaxBytes || n_s > kMaxBytes || n_kl > kMaxBytes)
        return fail(GDN_ERR_OVERFLOW, "%s: tensor sizes overflow", kFn);

    gdn::RecordArgs a{q, k, v, g, beta, state_in, mask, y, state_out, delta_log, k_log, g_log,
                      B, T, Hk, Hv, Dk, Dv, io_dtype, gqa_map, forced};
    const gdn::RowTiling til = gdn::record_tiling(a);
    uint64_t items;
    if (!mul_u64(&items, {B, Hv, Dv / static_cast<uint32_t>(til.rows()), static_cast<uint32_t>(til.threads)}) ||
        items > kMaxWorkItems)
        return fail(GDN_ERR_OVERFLOW, "%s: launch grid too large (B*Hv*Dv too large for one launch)", kFn);

    const void* a16[] = {q, k, v, state_in, y, state_out, delta_log, k_log};
    const char* a16n[] = {"q", "k", "v", "state_in", "y", "state_out", "delta_log", "k_log"};
    for (int i = 0; i < 8; ++i)
        if (a16[i] && !aligned(a16[i], 16))
            return fail(GDN_ERR_MISALIGNED, "%s: %s must be 16-byte aligned", kFn, a16n[i]);
    if (mask && !aligned(mask, 4)) return fail(GDN_ERR_MISALIGNED, "%s: mask must be 4-byte aligned", kFn);
    if (!aligned(g, e) || !aligned(beta, e) || (g_log && !aligned(g_log, e)))
        return fail(GDN_ERR_MISALIGNED, "%s: g, beta and g_log must be element-aligned", kFn);

    const Span ins[] = {{q, n_qk, "q"}, {k, n_qk, "k"}, {v, n_v, "v"}, {g, n_g, "g"},
                        {beta, n_g, "beta"}, {state_in, n_s, "state_in"}, {mask, mask ? n_m : 0, "mask"}};
    const Span outs[] = {{y, n_v, "y"}, {state_out, n_s, "state_out"},
                         {delta_log, delta_log ? n_v : 0, "delta_log"},
                         {k_log, k_log ? n_kl : 0, "k_log"}, {g_log, g_log ? n_g : 0, "g_log"}};
    constexpr int kOuts = 5;
    for (const Span& o : outs) {
        for (const Span& i : ins) {
            if (o.p == state_out && i.p == state_in && o.p == i.p) continue;   // exact in-place state
            if (overlaps(o, i)) return fail(GDN_ERR_ALIAS, "%s: %s overlaps %s", kFn, o.name, i.name);
        }
    }
    for (int i = 0; i < kOuts; ++i)
        for (int j = i + 1; j < kOuts; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(GDN_ERR_ALIAS, "%s: %s overlaps %s", kFn, outs[i].name, outs[j].name);

    return launch_status(gdn::launch_record(a, static_cast<hipStream_t>(stream)), kFn);
}

int replay_impl(const gdn_launch_choice* choice,
                const void* delta_log, const void* k_log, const void* g_log,
                const float* state_in, const uint32_t* mask, float* state_out,
                uint32_t B, uint32_t T_log, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                uint32_t accepted, int io_dtype, void* stream, const char* kFn) {
    if (!valid_dtype(io_dtype)) return fail(GDN_ERR_BAD_ENUM, "%s: unknown io_dtype %d", kFn, io_dtype);
    if (!delta_log || !k_log || !g_log || !state_in || !state_out)
        return fail(GDN_ERR_NULL, "%s: one of delta_log, k_log, g_log, state_in, state_out is NULL", kFn);
    if (B == 0 || T_log == 0 || Hv == 0 || Dk == 0 || Dv == 0)
        return fail(GDN_ERR_ZERO_DIM, "%s: zero-sized dimension in B=%u T_log=%u Hv=%u Dk=%u Dv=%u",
                    kFn, B, T_log, Hv, Dk, Dv);
    if (!gdn::dk_supported(Dk) || Dv % 16 != 0 || Dv > 1024)
        return fail(GDN_ERR_UNSUPPORTED_SHAPE,
                    "%s: no kernel for Dk=%u, Dv=%u (Dk in {32, 64, 128, 192, 256}; Dv a multiple "
                    "of 16, at most 1024)", kFn, Dk, Dv);
    gdn::RowTiling forced;
    {
        const int st = forced_tiling(choice, kFn, Dk, Dv, 1024u, &forced);
        if (st != GDN_OK) return st;
    }
    const int fold = choice ? choice->replay_fold : GDN_FOLD_AUTO;
    const uint32_t waves = choice ? choice->matrix_waves : 0u;
    if (fold != GDN_FOLD_AUTO && fold != GDN_FOLD_VALU && fold != GDN_FOLD_MATRIX)
        return fail(GDN_ERR_BAD_ENUM, "%s: unknown replay_fold %d", kFn, fold);
    if (waves != 0 && waves != 2 && waves != 4)
        return fail(GDN_ERR_BAD_ENUM, "%s: matrix_waves must be 0, 2 or 4 (got %u)", kFn, waves);

    const uint64_t e = io_bytes(io_dtype);
    uint64_t n_d, n_k, n_g, n_s, n_m;
    if (!mul_u64(&n_d, {B, T_log, Hv, Dv, e}) || !mul_u64(&n_k, {B, T_log, Hv, Dk, e}) ||
        !mul_u64(&n_g, {B, T_log, Hv, e}) || !mul_u64(&n_s, {B, Hv, Dv, Dk, 4}) ||
        !mul_u64(&n_m, {B, T_log, 4}) || n_d > kMaxBytes || n_k > kMaxBytes || n_s > kMaxBytes)
        return fail(GDN_ERR_OVERFLOW, "%s: tensor sizes overflow", kFn);

    gdn::ReplayArgs a{delta_log, k_log, g_log, state_in, mask, state_out,
                      B, T_log, Hv, Dk, Dv, accepted < T_log ? accepted : T_log, io_dtype,
                      forced, fold, waves};
    if (fold == GDN_FOLD_MATRIX && !gdn::replay_mfma_possible(a))
        return fail(GDN_ERR_UNSUPPORTED_SHAPE,
                    "%s: the matrix-core fold needs a 16-bit tape, Dv a multiple of 64 and at most "
                    "2^32 - 1 work-items (4 per state row)", kFn);
    if (!gdn::replay_mfma_applies(a)) {
        const gdn::RowTiling til = gdn::replay_tiling(a);
        uint64_t items;
        if (!mul_u64(&items, {B, Hv, Dv / static_cast<uint32_t>(til.rows()), static_cast<uint32_t>(til.threads)}) ||
            items > kMaxWorkItems)
            return fail(GDN_ERR_OVERFLOW, "%s: launch grid too large (B*Hv*Dv too large for one launch)", kFn);
    }

    const void* a16[] = {delta_log, k_log, state_in, state_out};
    const char* a16n[] = {"delta_log", "k_log", "state_in", "state_out"};
    for (int i = 0; i < 4; ++i)
        if (!aligned(a16[i], 16)) return fail(GDN_ERR_MISALIGNED, "%s: %s must be 16-byte aligned", kFn, a16n[i]);
    if (mask && !aligned(mask, 4)) return fail(GDN_ERR_MISALIGNED, "%s: mask must be 4-byte aligned", kFn);
    if (!aligned(g_log, e)) return fail(GDN_ERR_MISALIGNED, "%s: g_log must be element-aligned", kFn);

    const Span out{state_out, n_s, "state_out"};
    const Span ins[] = {{delta_log, n_d, "delta_log"}, {k_log, n_k, "k_log"}, {g_log, n_g, "g_log"},
                        {state_in, n_s, "state_in"}, {mask, mask ? n_m : 0, "mask"}};
    for (const Span& i : ins) {
        if (i.p == state_in && out.p == state_in) continue;                   // exact in-place state
        if (overlaps(out, i)) return fail(GDN_ERR_ALIAS, "%s: state_out overlaps %s", kFn, i.name);
    }

    return launch_status(gdn::launch_replay(a, static_cast<hipStream_t>(stream)), kFn);
}

}  // namespace

extern "C" {

int gdn_record(const void* q, const void* k, const void* v, const void* g, const void* beta,
               const float* state_in, const uint32_t* mask,
               void* y, float* state_out, void* delta_log, void* k_log, void* g_log,
               uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dk, uint32_t Dv,
               int io_dtype, int gqa_map, void* stream) {
    return record_impl(nullptr, q, k, v, g, beta, state_in, mask, y, state_out, delta_log, k_log, g_log,
                       B, T, Hk, Hv, Dk, Dv, io_dtype, gqa_map, stream, "gdn_record");
}

int gdn_record_debug(const gdn_launch_choice* choice,
                     const void* q, const void* k, const void* v, const void* g, const void* beta,
                     const float* state_in, const uint32_t* mask,
                     void* y, float* state_out, void* delta_log, void* k_log, void* g_log,
                     uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                     int io_dtype, int gqa_map, void* stream) {
    return record_impl(choice, q, k, v, g, beta, state_in, mask, y, state_out, delta_log, k_log, g_log,
                       B, T, Hk, Hv, Dk, Dv, io_dtype, gqa_map, stream, "gdn_record_debug");
}

int gdn_replay(const void* delta_log, const void* k_log, const void* g_log,
               const float* state_in, const uint32_t* mask, float* state_out,
               uint32_t B, uint32_t T_log, uint32_t Hv, uint32_t Dk, uint32_t Dv,
               uint32_t accepted, int io_dtype, void* stream) {
    return replay_impl(nullptr, delta_log, k_log, g_log, state_in, mask, state_out, B, T_log, Hv, Dk, Dv,
                       accepted, io_dtype, stream, "gdn_replay");
}

int gdn_replay_debug(const gdn_launch_choice* choice,
                     const void* delta_log, const void* k_log, const void* g_log,
                     const float* state_in, const uint32_t* mask, float* state_out,
                     uint32_t B, uint32_t T_log, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                     uint32_t accepted, int io_dtype, void* stream) {
    return replay_impl(choice, delta_log, k_log, g_log, state_in, mask, state_out, B, T_log, Hv, Dk, Dv,
                       accepted, io_dtype, stream, "gdn_replay_debug");
}

uint64_t gdn_prefill_workspace_size(uint32_t B, uint32_t T, uint32_t Hv) {
    return gdn::prefill_workspace_bytes(B, T, Hv);
}

}  // extern "C"

namespace {

// noalloc: the workspace is the library's own scratch area (workspace and
// workspace_bytes are ignored), looked up after validation.
int prefill_impl(bool noalloc, const void* q, const void* k, const void* v, const void* g, const void* beta,
                 const float* state_in, const uint32_t* mask,
                 void* y, float* state_out, void* delta_log, void* k_log, void* g_log,
                 void* workspace, uint64_t workspace_bytes,
                 uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                 int io_dtype, int gqa_map, void* stream, const char* kFn) {
    if (!valid_dtype(io_dtype)) return fail(GDN_ERR_BAD_ENUM, "%s: unknown io_dtype %d", kFn, io_dtype);
    if (!valid_map(gqa_map)) return fail(GDN_ERR_BAD_ENUM, "%s: unknown gqa_map %d", kFn, gqa_map);
    if (!q || !k || !v || !g || !beta || !state_in || !y || !state_out)
        return fail(GDN_ERR_NULL, "%s: one of q, k, v, g, beta, state_in, y, state_out is NULL", kFn);
    if (B == 0 || T == 0 || Hk == 0 || Hv == 0 || Dk == 0 || Dv == 0)
        return fail(GDN_ERR_ZERO_DIM, "%s: zero-sized dimension in B=%u T=%u Hk=%u Hv=%u Dk=%u Dv=%u",
                    kFn, B, T, Hk, Hv, Dk, Dv);
    if (Hv % Hk != 0)
        return fail(GDN_ERR_GQA_RATIO, "%s: %u value heads cannot share %u key heads evenly", kFn, Hv, Hk);
    if (!gdn::prefill_supported(Dk, Dv, io_dtype) || Dv > 1024)
        return fail(GDN_ERR_UNSUPPORTED_SHAPE,
                    "%s: needs bf16 or fp16 I/O, Dk = 128 or 192 and Dv a multiple of 16 up to 1024 "
                    "(got io_dtype=%d, Dk=%u, Dv=%u)", kFn, io_dtype, Dk, Dv);

    const uint64_t e = io_bytes(io_dtype);
    uint64_t n_qk, n_v, n_g, n_s, n_m, n_kl;
    if (!mul_u64(&n_qk, {B, T, Hk, Dk, e}) || !mul_u64(&n_v, {B, T, Hv, Dv, e}) ||
        !mul_u64(&n_g, {B, T, Hv, e}) || !mul_u64(&n_s, {B, Hv, Dv, Dk, 4}) || !mul_u64(&n_m, {B, T, 4}) ||
        !mul_u64(&n_kl, {B, T, Hv, Dk, e}) ||
        n_qk > kMaxBytes || n_v > kMaxBytes || n_s > kMaxBytes || n_kl > kMaxBytes)
        return fail(GDN_ERR_OVERFLOW, "%s: tensor sizes overflow", kFn);
    const uint64_t nchunks = (uint64_t(T) + 63) / 64;
    uint64_t prep_items, scan_items;
    if (!mul_u64(&prep_items, {B, Hv, nchunks, 256}) || prep_items > kMaxWorkItems ||
        !mul_u64(&scan_items, {B, Hv, Dv / 16, 512}) || scan_items > kMaxWorkItems)
        return fail(GDN_ERR_OVERFLOW, "%s: launch grid too large (split the batch)", kFn);
    const uint64_t need = gdn::prefill_workspace_bytes(B, T, Hv);
    if (noalloc) {
        if (need > gdn::kPrefillScratchBytes)
            return fail(GDN_ERR_WORKSPACE,
                        "%s: these sizes need %llu bytes of workspace; the library's scratch area holds "
                        "%llu (B*Hv*ceil(T/64) = %llu blocks, at most 2048): split the batch or the "
                        "heads, or call gdn_prefill with a workspace", kFn,
                        static_cast<unsigned long long>(need),
                        static_cast<unsigned long long>(gdn::kPrefillScratchBytes),
                        static_cast<unsigned long long>(need / 33280u));
        workspace = nullptr;
    } else if (!workspace || workspace_bytes < need) {
        return fail(GDN_ERR_WORKSPACE, "%s: workspace of %llu bytes needed, %llu given%s", kFn,
                    static_cast<unsigned long long>(need), static_cast<unsigned long long>(workspace_bytes),
                    workspace ? "" : " (NULL)");
    }

    const void* a16[] = {q, k, v, state_in, y, state_out, delta_log, k_log};
    const char* a16n[] = {"q", "k", "v", "state_in", "y", "state_out", "delta_log", "k_log"};
    for (int i = 0; i < 8; ++i)
        if (a16[i] && !aligned(a16[i], 16))
            return fail(GDN_ERR_MISALIGNED, "%s: %s must be 16-byte aligned", kFn, a16n[i]);
    if (!noalloc && !aligned(workspace, 256))
        return fail(GDN_ERR_MISALIGNED, "%s: workspace must be 256-byte aligned", kFn);
    if (mask && !aligned(mask, 4)) return fail(GDN_ERR_MISALIGNED, "%s: mask must be 4-byte aligned", kFn);
    if (!aligned(g, e) || !aligned(beta, e) || (g_log && !aligned(g_log, e)))
        return fail(GDN_ERR_MISALIGNED, "%s: g, beta and g_log must be element-aligned", kFn);

    const Span ins[] = {{q, n_qk, "q"}, {k, n_qk, "k"}, {v, n_v, "v"}, {g, n_g, "g"},
                        {beta, n_g, "beta"}, {state_in, n_s, "state_in"}, {mask, mask ? n_m : 0, "mask"}};
    const Span outs[] = {{y, n_v, "y"}, {state_out, n_s, "state_out"},
                         {delta_log, delta_log ? n_v : 0, "delta_log"},
                         {k_log, k_log ? n_kl : 0, "k_log"}, {g_log, g_log ? n_g : 0, "g_log"},
                         {workspace, noalloc ? 0 : need, "workspace"}};
    constexpr int kOuts = 6;
    for (const Span& o : outs) {
        for (const Span& i : ins) {
            if (o.p == state_out && i.p == state_in && o.p == i.p) continue;   // exact in-place state
            if (overlaps(o, i)) return fail(GDN_ERR_ALIAS, "%s: %s overlaps %s", kFn, o.name, i.name);
        }
    }
    for (int i = 0; i < kOuts; ++i)
        for (int j = i + 1; j < kOuts; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(GDN_ERR_ALIAS, "%s: %s overlaps %s", kFn, outs[i].name, outs[j].name);

    if (noalloc) {
        const hipError_t e = gdn::prefill_scratch(static_cast<hipStream_t>(stream), &workspace);
        if (e == hipErrorInvalidDevice)
            return fail(GDN_ERR_LAUNCH, "%s: the stream does not belong to the current device", kFn);
        if (e != hipSuccess)
            return fail(GDN_ERR_LAUNCH, "%s: cannot find the scratch area: %s", kFn, hipGetErrorString(e));
    }
    gdn::PrefillArgs a{q, k, v, g, beta, state_in, mask, y, state_out, delta_log, k_log, g_log, workspace,
                       B, T, Hk, Hv, Dk, Dv, io_dtype, gqa_map};
    return launch_status(gdn::launch_prefill(a, static_cast<hipStream_t>(stream)), kFn);
}

}  // namespace

extern "C" {

int gdn_prefill(const void* q, const void* k, const void* v, const void* g, const void* beta,
                const float* state_in, const uint32_t* mask,
                void* y, float* state_out, void* delta_log, void* k_log, void* g_log,
                void* workspace, uint64_t workspace_bytes,
                uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                int io_dtype, int gqa_map, void* stream) {
    return prefill_impl(false, q, k, v, g, beta, state_in, mask, y, state_out, delta_log, k_log, g_log,
                        workspace, workspace_bytes, B, T, Hk, Hv, Dk, Dv, io_dtype, gqa_map, stream,
                        "gdn_prefill");
}

int gdn_prefill_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                        const float* state_in, const uint32_t* mask,
                        void* y, float* state_out, void* delta_log, void* k_log, void* g_log,
                        uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                        int io_dtype, int gqa_map, void* stream) {
    return prefill_impl(true, q, k, v, g, beta, state_in, mask, y, state_out, delta_log, k_log, g_log,
                        nullptr, 0, B, T, Hk, Hv, Dk, Dv, io_dtype, gqa_map, stream, "gdn_prefill_noalloc");
}

int gqa_expand(const void* src, void* dst, uint32_t seq, uint32_t hg, uint32_t h, uint32_t k,
               int dtype, int gqa_map, void* stream) {
    static const char* kFn = "gqa_expand";
    if (!valid_dtype(dtype)) return fail(GDN_ERR_BAD_ENUM, "%s: unknown dtype %d", kFn, dtype);
    if (!valid_map(gqa_map)) return fail(GDN_ERR_BAD_ENUM, "%s: unknown gqa_map %d", kFn, gqa_map);
    if (!src || !dst) return fail(GDN_ERR_NULL, "%s: src or dst is NULL", kFn);
    if (seq == 0 || hg == 0 || h == 0 || k == 0)
        return fail(GDN_ERR_ZERO_DIM, "%s: zero-sized dimension in seq=%u hg=%u h=%u k=%u", kFn, seq, hg, h, k);
    if (h % hg != 0)
        return fail(GDN_ERR_GQA_RATIO, "%s: %u destination heads cannot be spread evenly over %u source heads",
                    kFn, h, hg);
    const uint64_t e = io_bytes(dtype);
    uint64_t n_src, n_dst;
    if (!mul_u64(&n_src, {seq, hg, k, e}) || !mul_u64(&n_dst, {seq, h, k, e}) || n_dst > kMaxBytes)
        return fail(GDN_ERR_OVERFLOW, "%s: seq*h*k overflows", kFn);
    if (!aligned(src, e) || !aligned(dst, e))
        return fail(GDN_ERR_MISALIGNED, "%s: src and dst must be element-aligned", kFn);
    if (overlaps(Span{src, n_src, "src"}, Span{dst, n_dst, "dst"}))
        return fail(GDN_ERR_ALIAS, "%s: dst overlaps src", kFn);
    gdn::ExpandArgs a{src, dst, seq, hg, h, k, static_cast<uint32_t>(e), gqa_map};
    return launch_status(gdn::launch_expand(a, static_cast<hipStream_t>(stream)), kFn);
}

int rms_norm_bf16(const float* x, const uint16_t* weight, float* out, uint32_t n_tokens,
                  uint32_t dim, float eps, void* stream) {
    static const char* kFn = "rms_norm_bf16";
    if (!x || !weight || !out) return fail(GDN_ERR_NULL, "%s: x, weight and out must be non-NULL", kFn);
    if (n_tokens == 0 || dim == 0) return fail(GDN_ERR_ZERO_DIM, "%s: n_tokens and dim must be > 0", kFn);
    uint64_t n_x;
    if (!mul_u64(&n_x, {n_tokens, dim, 4}) || n_x > kMaxBytes)
        return fail(GDN_ERR_OVERFLOW, "%s: n_tokens*dim overflows", kFn);
    if (!aligned(x, 4) || !aligned(out, 4) || !aligned(weight, 2))
        return fail(GDN_ERR_MISALIGNED, "%s: x and out must be 4-byte aligned, weight 2-byte", kFn);
    const Span sx{x, n_x, "x"}, so{out, n_x, "out"}, sw{weight, uint64_t(dim) * 2, "weight"};
    if ((out != x && overlaps(so, sx)) || overlaps(so, sw))
        return fail(GDN_ERR_ALIAS, "%s: out overlaps x (other than exactly) or the weight", kFn);
    gdn::RmsNormArgs a{x, weight, out, n_tokens, dim, eps};
    return launch_status(gdn::launch_rms_norm(a, static_cast<hipStream_t>(stream)), kFn);
}

}  // extern "C"
