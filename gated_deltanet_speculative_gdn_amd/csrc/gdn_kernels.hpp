// gdn_kernels.hpp -- kernel parameter blocks and launchers (internal to the
// library; the public interface is include/gdn_replay.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_divide.hpp"
#include "gdn_replay.h"

namespace gdn {

// One layer's verify (or native snapshot window). Passed by value as the
// kernel argument block.
struct VerifyParams {
    const void* state;        // layer pool [slots][HV][V][K]
    float* rec;               // layer record pool [rec_slots][HV][rec_stride]
    void* snap;               // native only: [rows][HV][T][V][K]
    const int32_t* state_slot;
    const int32_t* rec_slot;  // verify only
    const int32_t* tok_start;
    const int32_t* win_len;
    const int32_t* rec_base;  // verify only, may be null
    const uint16_t* q; int64_t q_ts, q_hs;
    const uint16_t* k; int64_t k_ts, k_hs;
    const uint16_t* v; int64_t v_ts, v_hs;
    const float* a_log; const float* beta; int64_t g_ts;   // log-gate and beta, or raw a and b
    const float* A_log; const float* dt_bias;               // raw gates only: per value head
    void* out; int64_t o_ts, o_hs;                          // fp32 or bf16 [tokens][HV][V]
    int64_t num_tokens;
    int64_t rec_stride;       // floats per (record slot, value head)
    int32_t* err;
    int32_t num_rows, hv, group, num_slots, num_rec_slots, T;
    Divider div_hv;           // division by hv
    float scale;
    bool raw_gates;           // gates from raw a, b with A_log, dt_bias
    bool out_bf16;            // outputs rounded to bf16 (nearest even)
    bool payload;             // payload records (k, v, gate, beta) instead of corrections
    bool channel;             // one decay per key channel: a_log is [tokens][HV][K] with
    int64_t a_ts;             //   token stride a_ts; records hold alpha[T][K] for the gate
};

// Short-conv state compaction, run by extra workgroups of the commit launch:
// one 16-byte column piece per thread, one workgroup per this many pieces.
constexpr int kConvPiecesPerWg = 256;
struct ConvParams {
    void* state[GDN_MAX_LAYERS];        // [slots][state_len][row_bytes]
    const void* x[GDN_MAX_LAYERS];      // [tokens][x_tok_bytes]
    const int32_t* tok_start;
    int64_t row_bytes;                  // bytes per state row, a multiple of 16
    int64_t x_tok_bytes;                // bytes between tokens of x, a multiple of 16
    int64_t num_tokens;
    int32_t state_len, num_slots;
    int32_t pieces;                     // 16-byte pieces per row
    int32_t wgs_per_row;                // workgroups per (layer, row)
    Divider div_wpr;                    // division by wgs_per_row
};

// The all-layer commit.
struct CommitParams {
    void* state[GDN_MAX_LAYERS];
    const float* rec[GDN_MAX_LAYERS];
    const int32_t* src;
    const int32_t* dst;
    const int32_t* rec_slot;
    const int32_t* n;
    const int32_t* bnd_len;   // align mode only
    const int32_t* bnd_slot;
    int32_t* err;
    int64_t rec_stride;
    int32_t num_layers, num_rows, hv, num_slots, num_rec_slots, T;
    Divider div_hv, div_rows; // division by hv and num_rows
    bool payload;             // payload records: the replay recomputes the corrections
    bool channel;             // per-channel decay records: alpha[T][K] in place of the gate
    int64_t ssm_wgs;          // workgroups of the state replay (after the conv's, below)
    int64_t conv_wgs;         // workgroups of the conv compaction (0 = none); they come first
                              // in the grid, their count padded to a multiple of the XCD count
    ConvParams conv;
};

// The native baseline's accepted-state copy.
struct AcceptParams {
    void* state[GDN_MAX_LAYERS];
    const void* snap[GDN_MAX_LAYERS];
    const int32_t* dst;
    const int32_t* n;
    int32_t* err;
    int32_t num_layers, num_rows, hv, num_slots, T;
    Divider div_hv, div_rows;
};

struct PlanParams {
    const int32_t* p0;
    const int32_t* n;
    const int32_t* table;
    int64_t table_stride;
    int32_t* src;
    int32_t* dst;
    int32_t* bnd_len;
    int32_t* bnd_slot;
    int32_t* err;
    int32_t num_rows, cols, block, max_n;
};

constexpr int kMaxRecTokens = GDN_MAX_REC_TOKENS;

// Verify launch shape: rows of a head each thread holds and threads per
// workgroup; a workgroup covers threads/8 * R rows. Windows of up to 4
// positions (the MTP shape) run 512-thread workgroups, one per head (bf16
// pools 3.4% and fp32 pools 0.6% faster than two 256-thread workgroups per
// head); longer windows, whose LDS staging is larger, run two 256-thread
// workgroups per head. One and four rows per thread measured no faster.
constexpr int kVerifyRowsPerThread = 2;
constexpr int kVerifyThreadsShort = 512;   // windows of up to 4 positions
constexpr int kVerifyThreads = 256;        // longer windows
// Commit: workgroups per head for fp32 and bf16 pools (8 KiB of state per
// workgroup streams best for both, at every record capacity, with the
// token-by-token replay; one workgroup per head measured slower); whether
// workgroup ids are remapped XCD-contiguous. State loads and stores are always
// nontemporal (cached streams measured slower).
constexpr int kCommitSplitF32 = 8;
constexpr int kCommitSplitBf16 = 4;
constexpr bool kCommitXcdRemap = true;
// The dispatch packet counts a launch's work-items (workgroups x threads) in 32
// bits, so one launch of 256-thread workgroups holds at most this many. The
// all-layer commit issues consecutive launches over runs of whole layers when
// its grid would exceed it (fp32 pools: beyond 2^21 (layer, row, head) triples,
// 137 GB of source state); one layer must fit in one launch.
constexpr int64_t kCommitThreads = 256;
constexpr int64_t kMaxLaunchWgs = (int64_t)0xFFFFFFFFu / kCommitThreads;
// Verify: a layer's launch is rows x value heads x 512 work-items (one 512-thread
// workgroup or two 256-thread ones per head).
constexpr int64_t kVerifyItemsPerHead = 512;

// Launchers: return the hipError_t of the launch.
hipError_t launch_verify(const VerifyParams& p, bool bf16_state, hipStream_t s);
hipError_t launch_native_window(const VerifyParams& p, bool bf16_state, hipStream_t s);
hipError_t launch_commit(const CommitParams& p, bool bf16_state, bool align, hipStream_t s);
hipError_t launch_native_accept(const AcceptParams& p, bool bf16_state, hipStream_t s);
hipError_t launch_align_plan(const PlanParams& p, hipStream_t s);

inline size_t commit_lds_bytes(int T, bool channel = false)
{
    return sizeof(float) * ((channel ? 3 : 2) * (size_t)T * 128 + 2 * (size_t)T);
}

}  // namespace gdn
