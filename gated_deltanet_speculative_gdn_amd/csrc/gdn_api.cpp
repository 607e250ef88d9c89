// gdn_api.cpp -- the C ABI declared in include/gdn_replay.h: argument
// validation, kernel parameter packing and launch. Validation finishes before
// any HIP call, so a rejected call touches neither the device nor the stream
// ([vLLM] RecoverSSM PR, Test Plan: malformed-input rejection).
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "gdn_kernels.hpp"
#include "gdn_replay.h"

namespace {

using namespace gdn;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int32_t check_pools(const gdn_pools* p)
{
    if (!p) return GDN_ERR_NULL;
    if (p->num_layers < 1 || p->num_layers > GDN_MAX_LAYERS) return GDN_ERR_SHAPE;
    if (p->head_k_dim != GDN_HEAD_DIM || p->head_v_dim != GDN_HEAD_DIM) return GDN_ERR_SHAPE;
    if (p->num_v_heads < 1 || p->num_k_heads < 1 || p->num_v_heads % p->num_k_heads)
        return GDN_ERR_SHAPE;
    if (p->num_v_heads > 4096) return GDN_ERR_SHAPE;
    if (p->state_dtype != GDN_STATE_F32 && p->state_dtype != GDN_STATE_BF16) return GDN_ERR_DTYPE;
    if (p->num_state_slots < 1 || p->num_rec_slots < 1) return GDN_ERR_SHAPE;
    if (p->rec_tokens < 1 || p->rec_tokens > GDN_MAX_REC_TOKENS) return GDN_ERR_SHAPE;
    if (p->record_kind != GDN_RECORD_CORRECTION && p->record_kind != GDN_RECORD_PAYLOAD &&
        p->record_kind != GDN_RECORD_CHANNEL)
        return GDN_ERR_SHAPE;
    return GDN_OK;
}

int32_t check_layer_ptrs(const gdn_pools* p, int32_t layer, bool need_rec)
{
    if (!p->state[layer] || (need_rec && !p->rec[layer])) return GDN_ERR_NULL;
    if (!aligned16(p->state[layer]) || (need_rec && !aligned16(p->rec[layer])))
        return GDN_ERR_ALIGN;
    return GDN_OK;
}

int32_t check_io(const gdn_verify_io* io)
{
    if (!io) return GDN_ERR_NULL;
    if (!io->q || !io->k || !io->v || !io->a || !io->b || !io->out) return GDN_ERR_NULL;
    if (io->gate_mode != GDN_GATE_LOG && io->gate_mode != GDN_GATE_RAW &&
        io->gate_mode != GDN_GATE_CHANNEL)
        return GDN_ERR_SHAPE;
    if (io->out_dtype != GDN_OUT_F32 && io->out_dtype != GDN_OUT_BF16) return GDN_ERR_DTYPE;
    if (io->gate_mode == GDN_GATE_RAW && (!io->A_log || !io->dt_bias)) return GDN_ERR_NULL;
    if (io->num_tokens < 0 || io->gate_tok_stride < 0) return GDN_ERR_SHAPE;
    if (io->q_tok_stride < 0 || io->q_head_stride < 0 || io->k_tok_stride < 0 ||
        io->k_head_stride < 0 || io->v_tok_stride < 0 || io->v_head_stride < 0 ||
        io->out_tok_stride < 0 || io->out_head_stride < 0)
        return GDN_ERR_SHAPE;
    // 16-byte vector access: bf16 input rows need strides in multiples of 8
    // elements; output pieces are 4 elements (16 bytes fp32, 8 bytes bf16).
    if (!aligned16(io->q) || !aligned16(io->k) || !aligned16(io->v)) return GDN_ERR_ALIGN;
    if (io->out_dtype == GDN_OUT_F32 ? !aligned16(io->out) : ((uintptr_t)io->out & 7u) != 0)
        return GDN_ERR_ALIGN;
    if ((io->q_tok_stride | io->q_head_stride | io->k_tok_stride | io->k_head_stride |
         io->v_tok_stride | io->v_head_stride) & 7)
        return GDN_ERR_ALIGN;
    if ((io->out_tok_stride | io->out_head_stride) & 3) return GDN_ERR_ALIGN;
    if (((uintptr_t)io->a & 3u) || ((uintptr_t)io->b & 3u)) return GDN_ERR_ALIGN;
    if (io->gate_mode == GDN_GATE_RAW && (((uintptr_t)io->A_log & 3u) || ((uintptr_t)io->dt_bias & 3u)))
        return GDN_ERR_ALIGN;
    if (io->gate_mode == GDN_GATE_CHANNEL) {
        if (io->decay_tok_stride < 0) return GDN_ERR_SHAPE;
        if (!aligned16(io->a) || (io->decay_tok_stride & 3)) return GDN_ERR_ALIGN;
    }
    return GDN_OK;
}

int64_t conv_elem_bytes(const gdn_conv_pools* c) { return c->dtype == GDN_STATE_BF16 ? 2 : 4; }
int64_t conv_row_bytes(const gdn_conv_pools* c) { return (int64_t)c->channels * conv_elem_bytes(c); }

int32_t check_conv(const gdn_conv_pools* c)
{
    if (c->num_layers < 1 || c->num_layers > GDN_MAX_LAYERS) return GDN_ERR_SHAPE;
    if (c->dtype != GDN_STATE_F32 && c->dtype != GDN_STATE_BF16) return GDN_ERR_DTYPE;
    if (c->channels < 1 || c->state_len < 1 || c->state_len > GDN_MAX_CONV_STATE ||
        c->num_slots < 1 || c->num_tokens < 0 || c->x_tok_stride < c->channels)
        return GDN_ERR_SHAPE;
    if ((int64_t)c->channels * conv_elem_bytes(c) / 16 > INT32_MAX) return GDN_ERR_SHAPE;
    if ((conv_row_bytes(c) & 15) || ((c->x_tok_stride * conv_elem_bytes(c)) & 15))
        return GDN_ERR_ALIGN;
    for (int32_t l = 0; l < c->num_layers; ++l) {
        if (!c->state[l] || !c->x[l]) return GDN_ERR_NULL;
        if (!aligned16(c->state[l]) || !aligned16(c->x[l])) return GDN_ERR_ALIGN;
    }
    return GDN_OK;
}

void fill_io(VerifyParams& v, const gdn_verify_io* io)
{
    v.q = io->q; v.q_ts = io->q_tok_stride; v.q_hs = io->q_head_stride;
    v.k = io->k; v.k_ts = io->k_tok_stride; v.k_hs = io->k_head_stride;
    v.v = io->v; v.v_ts = io->v_tok_stride; v.v_hs = io->v_head_stride;
    v.a_log = io->a; v.beta = io->b; v.g_ts = io->gate_tok_stride;
    v.raw_gates = io->gate_mode == GDN_GATE_RAW;
    v.A_log = io->A_log; v.dt_bias = io->dt_bias;
    v.out = io->out; v.o_ts = io->out_tok_stride; v.o_hs = io->out_head_stride;
    v.out_bf16 = io->out_dtype == GDN_OUT_BF16;
    v.channel = io->gate_mode == GDN_GATE_CHANNEL;
    v.a_ts = io->decay_tok_stride;
    v.num_tokens = io->num_tokens;
    v.scale = io->scale;
}

int32_t launched(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

}  // namespace

extern "C" {

int64_t gdn_rec_stride(int32_t rec_tokens)
{
    if (rec_tokens < 1) return 0;
    return (int64_t)rec_tokens * (2 * GDN_HEAD_DIM) + (((int64_t)rec_tokens + 3) & ~(int64_t)3);
}

int64_t gdn_record_stride(int32_t rec_tokens, int32_t record_kind)
{
    if (rec_tokens < 1) return 0;
    if (record_kind == GDN_RECORD_CORRECTION) return gdn_rec_stride(rec_tokens);
    if (record_kind == GDN_RECORD_CHANNEL) return (int64_t)rec_tokens * 3 * GDN_HEAD_DIM;
    if (record_kind != GDN_RECORD_PAYLOAD) return 0;
    const int64_t bytes = (int64_t)rec_tokens * (2 * GDN_HEAD_DIM * 2 + 8);
    return ((bytes + 15) & ~(int64_t)15) / 4;
}

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(int32_t s)
{
    switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "a size or index argument is out of range";
    case GDN_ERR_DTYPE: return "unsupported state or output dtype";
    case GDN_ERR_ALIGN: return "a pointer or stride breaks the 16-byte alignment rule";
    case GDN_ERR_LAUNCH: return "the HIP kernel launch failed";
    default: return "unknown status";
    }
}

int32_t gdn_verify(const gdn_pools* pools, int32_t layer, int32_t num_rows,
                   const int32_t* state_slot, const int32_t* rec_slot,
                   const int32_t* tok_start, const int32_t* win_len,
                   const int32_t* rec_base, const gdn_verify_io* io,
                   int32_t* err_flags, void* stream)
{
    int32_t st = check_pools(pools);
    if (st) return st;
    if (layer < 0 || layer >= pools->num_layers || num_rows < 0) return GDN_ERR_SHAPE;
    if ((int64_t)num_rows * pools->num_v_heads * kVerifyItemsPerHead > (int64_t)0xFFFFFFFFu)
        return GDN_ERR_SHAPE;
    if ((st = check_layer_ptrs(pools, layer, true))) return st;
    if ((st = check_io(io))) return st;
    if (!state_slot || !rec_slot || !tok_start || !win_len) return GDN_ERR_NULL;
    if (rec_base && pools->record_kind == GDN_RECORD_PAYLOAD) return GDN_ERR_SHAPE;
    if ((pools->record_kind == GDN_RECORD_CHANNEL) != (io->gate_mode == GDN_GATE_CHANNEL))
        return GDN_ERR_SHAPE;
    if (io->gate_mode == GDN_GATE_CHANNEL &&
        io->decay_tok_stride < (int64_t)pools->num_v_heads * GDN_HEAD_DIM)
        return GDN_ERR_SHAPE;
    if (num_rows == 0) return GDN_OK;

    VerifyParams v;
    memset(&v, 0, sizeof(v));
    v.state = pools->state[layer];
    v.rec = pools->rec[layer];
    v.payload = pools->record_kind == GDN_RECORD_PAYLOAD;
    v.state_slot = state_slot;
    v.rec_slot = rec_slot;
    v.tok_start = tok_start;
    v.win_len = win_len;
    v.rec_base = rec_base;
    fill_io(v, io);
    v.rec_stride = gdn_record_stride(pools->rec_tokens, pools->record_kind);
    v.err = err_flags;
    v.num_rows = num_rows;
    v.hv = pools->num_v_heads;
    v.group = pools->num_v_heads / pools->num_k_heads;
    v.num_slots = pools->num_state_slots;
    v.num_rec_slots = pools->num_rec_slots;
    v.T = pools->rec_tokens;
    v.div_hv = make_divider((uint32_t)v.hv);
    return launched(launch_verify(v, pools->state_dtype == GDN_STATE_BF16, (hipStream_t)stream));
}

int32_t gdn_native_window(const gdn_pools* pools, int32_t layer, int32_t num_rows,
                          const int32_t* state_slot, const int32_t* tok_start,
                          const int32_t* win_len, const gdn_verify_io* io, void* snap,
                          int32_t* err_flags, void* stream)
{
    int32_t st = check_pools(pools);
    if (st) return st;
    if (layer < 0 || layer >= pools->num_layers || num_rows < 0) return GDN_ERR_SHAPE;
    if ((int64_t)num_rows * pools->num_v_heads * kVerifyItemsPerHead > (int64_t)0xFFFFFFFFu)
        return GDN_ERR_SHAPE;
    if ((st = check_layer_ptrs(pools, layer, false))) return st;
    if ((st = check_io(io))) return st;
    if (!state_slot || !tok_start || !win_len || !snap) return GDN_ERR_NULL;
    if (!aligned16(snap)) return GDN_ERR_ALIGN;
    if (io->gate_mode == GDN_GATE_CHANNEL &&
        io->decay_tok_stride < (int64_t)pools->num_v_heads * GDN_HEAD_DIM)
        return GDN_ERR_SHAPE;
    if (num_rows == 0) return GDN_OK;

    VerifyParams v;
    memset(&v, 0, sizeof(v));
    v.state = pools->state[layer];
    v.snap = snap;
    v.state_slot = state_slot;
    v.tok_start = tok_start;
    v.win_len = win_len;
    fill_io(v, io);
    v.err = err_flags;
    v.num_rows = num_rows;
    v.hv = pools->num_v_heads;
    v.group = pools->num_v_heads / pools->num_k_heads;
    v.num_slots = pools->num_state_slots;
    v.num_rec_slots = pools->num_rec_slots;
    v.T = pools->rec_tokens;
    v.div_hv = make_divider((uint32_t)v.hv);
    return launched(
        launch_native_window(v, pools->state_dtype == GDN_STATE_BF16, (hipStream_t)stream));
}

int32_t gdn_commit_all_layers_conv(const gdn_pools* pools, const gdn_conv_pools* conv,
                                   int32_t num_rows, const int32_t* src_slot,
                                   const int32_t* dst_slot, const int32_t* rec_slot,
                                   const int32_t* n_accept, const int32_t* bnd_len,
                                   const int32_t* bnd_slot, const int32_t* conv_tok_start,
                                   int32_t* err_flags, void* stream)
{
    int32_t st;
    if (!pools && !conv) return GDN_ERR_NULL;
    if (pools) {
        if ((st = check_pools(pools))) return st;
        for (int32_t l = 0; l < pools->num_layers; ++l)
            if ((st = check_layer_ptrs(pools, l, true))) return st;
        if (!rec_slot) return GDN_ERR_NULL;
    }
    if (conv) {
        if ((st = check_conv(conv))) return st;
        if (pools && conv->num_layers != pools->num_layers) return GDN_ERR_SHAPE;
        if (!conv_tok_start) return GDN_ERR_NULL;
    }
    if (num_rows < 0) return GDN_ERR_SHAPE;
    const int32_t layers = pools ? pools->num_layers : conv->num_layers;
    // one layer's workgroups must fit in one launch (the launcher splits the
    // layers over several launches when all of them do not)
    int64_t layer_wgs = 0;
    if (pools) layer_wgs += (int64_t)num_rows * pools->num_v_heads * kCommitSplitF32;
    int64_t conv_per_row = 0;
    if (conv) {
        const int64_t pieces = conv_row_bytes(conv) / 16;
        conv_per_row = (pieces + kConvPiecesPerWg - 1) / kConvPiecesPerWg;
        layer_wgs += (int64_t)num_rows * conv_per_row;
    }
    if (layer_wgs > kMaxLaunchWgs - 8) return GDN_ERR_SHAPE;
    if (!src_slot || !dst_slot || !n_accept) return GDN_ERR_NULL;
    if ((bnd_len == nullptr) != (bnd_slot == nullptr)) return GDN_ERR_NULL;
    if (num_rows == 0) return GDN_OK;

    CommitParams c;
    memset(&c, 0, sizeof(c));
    c.src = src_slot;
    c.dst = dst_slot;
    c.n = n_accept;
    c.bnd_len = bnd_len;
    c.bnd_slot = bnd_slot;
    c.err = err_flags;
    c.num_layers = layers;
    c.num_rows = num_rows;
    if (pools) {
        for (int32_t l = 0; l < layers; ++l) {
            c.state[l] = pools->state[l];
            c.rec[l] = pools->rec[l];
        }
        c.rec_slot = rec_slot;
        c.rec_stride = gdn_record_stride(pools->rec_tokens, pools->record_kind);
        c.payload = pools->record_kind == GDN_RECORD_PAYLOAD;
        c.channel = pools->record_kind == GDN_RECORD_CHANNEL;
        c.hv = pools->num_v_heads;
        c.num_slots = pools->num_state_slots;
        c.num_rec_slots = pools->num_rec_slots;
        c.T = pools->rec_tokens;
    }
    if (conv) {
        ConvParams& v = c.conv;
        for (int32_t l = 0; l < layers; ++l) {
            v.state[l] = conv->state[l];
            v.x[l] = conv->x[l];
        }
        v.tok_start = conv_tok_start;
        v.row_bytes = conv_row_bytes(conv);
        v.x_tok_bytes = conv->x_tok_stride * conv_elem_bytes(conv);
        v.num_tokens = conv->num_tokens;
        v.state_len = conv->state_len;
        v.num_slots = conv->num_slots;
        v.pieces = (int32_t)(v.row_bytes / 16);
        v.wgs_per_row = (int32_t)conv_per_row;
        v.div_wpr = make_divider((uint32_t)conv_per_row);
        c.conv_wgs = (int64_t)num_rows * layers * conv_per_row;
    }
    c.div_hv = make_divider((uint32_t)c.hv);
    c.div_rows = make_divider((uint32_t)num_rows);
    const bool bf16 = pools && pools->state_dtype == GDN_STATE_BF16;
    return launched(launch_commit(c, bf16, bnd_len != nullptr, (hipStream_t)stream));
}

int32_t gdn_commit_all_layers(const gdn_pools* pools, int32_t num_rows,
                              const int32_t* src_slot, const int32_t* dst_slot,
                              const int32_t* rec_slot, const int32_t* n_accept,
                              const int32_t* bnd_len, const int32_t* bnd_slot,
                              int32_t* err_flags, void* stream)
{
    if (!pools) return GDN_ERR_NULL;
    return gdn_commit_all_layers_conv(pools, nullptr, num_rows, src_slot, dst_slot, rec_slot,
                                      n_accept, bnd_len, bnd_slot, nullptr, err_flags, stream);
}

int32_t gdn_native_accept(const gdn_pools* pools, void* const* snap_layers, int32_t num_rows,
                          const int32_t* dst_slot, const int32_t* n_accept, int32_t* err_flags,
                          void* stream)
{
    int32_t st = check_pools(pools);
    if (st) return st;
    if (num_rows < 0) return GDN_ERR_SHAPE;
    if ((int64_t)num_rows * pools->num_v_heads * pools->num_layers > kMaxLaunchWgs)
        return GDN_ERR_SHAPE;
    if (!snap_layers || !dst_slot || !n_accept) return GDN_ERR_NULL;
    for (int32_t l = 0; l < pools->num_layers; ++l) {
        if ((st = check_layer_ptrs(pools, l, false))) return st;
        if (!snap_layers[l]) return GDN_ERR_NULL;
        if (!aligned16(snap_layers[l])) return GDN_ERR_ALIGN;
    }
    if (num_rows == 0) return GDN_OK;

    AcceptParams a;
    memset(&a, 0, sizeof(a));
    for (int32_t l = 0; l < pools->num_layers; ++l) {
        a.state[l] = pools->state[l];
        a.snap[l] = snap_layers[l];
    }
    a.dst = dst_slot;
    a.n = n_accept;
    a.err = err_flags;
    a.num_layers = pools->num_layers;
    a.num_rows = num_rows;
    a.hv = pools->num_v_heads;
    a.num_slots = pools->num_state_slots;
    a.T = pools->rec_tokens;
    a.div_hv = make_divider((uint32_t)a.hv);
    a.div_rows = make_divider((uint32_t)num_rows);
    return launched(
        launch_native_accept(a, pools->state_dtype == GDN_STATE_BF16, (hipStream_t)stream));
}

int32_t gdn_align_plan(int32_t num_rows, const int32_t* num_computed, const int32_t* n_accept,
                       const int32_t* block_table, int64_t bt_row_stride, int32_t bt_cols,
                       int32_t block_size, int32_t max_accept, int32_t* src_slot,
                       int32_t* dst_slot, int32_t* bnd_len, int32_t* bnd_slot,
                       int32_t* err_flags, void* stream)
{
    if (num_rows < 0 || block_size < 1 || max_accept < 0 || bt_cols < 1 || bt_row_stride < bt_cols)
        return GDN_ERR_SHAPE;
    if (!num_computed || !n_accept || !block_table || !src_slot || !dst_slot || !bnd_len ||
        !bnd_slot)
        return GDN_ERR_NULL;
    if (num_rows == 0) return GDN_OK;
    PlanParams p;
    p.p0 = num_computed;
    p.n = n_accept;
    p.table = block_table;
    p.table_stride = bt_row_stride;
    p.src = src_slot;
    p.dst = dst_slot;
    p.bnd_len = bnd_len;
    p.bnd_slot = bnd_slot;
    p.err = err_flags;
    p.num_rows = num_rows;
    p.cols = bt_cols;
    p.block = block_size;
    p.max_n = max_accept;
    return launched(launch_align_plan(p, (hipStream_t)stream));
}

}  // extern "C"
